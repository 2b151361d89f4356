"""Gates per key channel (DN_GATE_PER_KEY; the nnterp page's ChannelGates, the KDA
variant) on the HIP path against the fp64 oracle (needs an MI355X).

g is ``[B, T, Hv, Dk]`` (prefill) or ``[N, Hv, Dk]`` (decode); key channel x of the state
keeps exp(g_t[x]) at token t.  Bar as for every parity test: relative L2 over the whole
tensor, 1e-4 for fp32 inputs, 1e-2 for bf16 inputs, outputs and final states.
"""
import sys

import numpy as np
import pytest
import torch

import delta_rule_recurrent_chunked_amd as dn
from synth import make_case
from tests.gpu_util import host, rel_l2, run_oracle, to_inputs, tol

pytestmark = pytest.mark.gpu


def _say(*a):
    print(*a, flush=True)
    sys.stdout.flush()


def _oracle(x, scale=1.0, qk_l2norm=False):
    import oracle
    f = x.f64()
    return oracle.recurrent(f["q"], f["k"], f["v"], f["beta"], f["g"], f["init"],
                            x.cu_seqlens, scale=scale, qk_l2norm=qk_l2norm)


def _check(x, o, s, o_ref, s_ref):
    eo, es = rel_l2(o, o_ref), rel_l2(s, s_ref)
    _say(f"  {x.name}: rel_l2 o={eo:.2e} state={es:.2e} (bar {tol(x):.0e})")
    assert np.all(np.isfinite(o)) and np.all(np.isfinite(s))
    assert eo <= tol(x) and es <= tol(x)


CASES = {
    "f32_d16": dict(B=1, T=64, Hqk=2, Dk=16, dtype="f32", g_scale=0.2),
    "f32_dk64_dv32_ragged": dict(B=2, T=150, Hqk=2, Dk=64, Dv=32, dtype="f32", g_scale=0.1,
                                 init_std=0.3, beta_scale=2.0),
    "f32_dk32_dv128_gqa": dict(B=1, T=77, Hqk=1, Hv=3, Dk=32, Dv=128, dtype="f32", g_scale=0.5,
                               init_std=1.0),
    "bf16_d128_packed_gqa": dict(B=1, Hqk=2, Hv=4, Dk=128, dtype="bf16",
                                 seqlens=[70, 0, 1, 64, 129, 0], g_scale=0.05, init_std=0.02,
                                 beta_scale=2.0),
    "bf16_d128_long": dict(B=1, T=700, Hqk=1, Hv=2, Dk=128, dtype="bf16", g_scale=0.1,
                           init_std=0.02),
    # decay strong enough that chunks fall below exp(-60): the per-pair exponential form
    "f32_strong_decay": dict(B=1, T=80, Hqk=2, Dk=32, dtype="f32", g_scale=5.0, init_std=0.3),
    # the matrix-core kernel: 16-token blocks that decay by more than exp(-60) take exact
    # diagonal tiles, the rest (and every block at the milder rate) the factored form
    "bf16_d128_strong_decay": dict(B=1, T=300, Hqk=2, Dk=128, dtype="bf16", g_scale=3.0,
                                   init_std=0.3),
    "bf16_d128_every_block_exact": dict(B=1, T=100, Hqk=2, Dk=128, dtype="bf16", g_scale=5.0,
                                        init_std=0.3),
    "bf16_d128_mixed_decay": dict(B=2, T=200, Hqk=1, Hv=2, Dk=128, dtype="bf16", g_scale=0.9,
                                  init_std=0.3, beta_scale=2.0),
    "bf16_d128_dv64": dict(B=1, T=190, Hqk=2, Hv=2, Dk=128, Dv=64, dtype="bf16", g_scale=0.2,
                           init_std=0.1),
    # bf16 sizes the matrix-core kernel does not take run the vector-ALU kernel
    "bf16_dk64_vector_path": dict(B=1, T=100, Hqk=2, Dk=64, Dv=64, dtype="bf16", g_scale=0.2,
                                  init_std=0.1),
}


@pytest.mark.parametrize("name", sorted(CASES))
def test_prefill_channel_gates(name):
    _say(f"channel gates prefill {name}")
    x = make_case(seed=21, name=name, g_per_key=True, **CASES[name])
    d = to_inputs(x)
    o, s = dn.chunk_fwd(d["q"], d["k"], d["v"], d["beta"], d["g"], d["init"],
                        cu_seqlens=d["cu"], scale=0.75)
    torch.cuda.synchronize()
    o_ref, s_ref = _oracle(x, 0.75)
    _check(x, host(o), host(s), o_ref, s_ref)


@pytest.mark.parametrize("chunk", [16, 32, 64])
def test_channel_gates_chunk_sizes(chunk):
    """The vector-ALU kernel at three chunk sizes (fp32, Dk = 64)."""
    _say(f"channel gates chunk {chunk}")
    x = make_case(B=1, T=100, Hqk=2, Dk=64, dtype="f32", g_scale=0.2, init_std=0.1, seed=22,
                  name=f"chunk{chunk}", g_per_key=True)
    d = to_inputs(x)
    o, s = dn.chunk_fwd(d["q"], d["k"], d["v"], d["beta"], d["g"], d["init"], chunk_size=chunk)
    torch.cuda.synchronize()
    o_ref, s_ref = _oracle(x)
    _check(x, host(o), host(s), o_ref, s_ref)


def test_channel_gates_with_in_call_normalisation():
    _say("channel gates + in-call q/k normalisation")
    x = make_case(B=1, T=130, Hqk=2, Hv=2, Dk=128, dtype="bf16", g_scale=0.1, init_std=0.02,
                  seed=23, name="chg_norm", g_per_key=True, qk_raw=True)
    d = to_inputs(x)
    o, s = dn.chunk_fwd(d["q"], d["k"], d["v"], d["beta"], d["g"], d["init"], qk_l2norm=True)
    torch.cuda.synchronize()
    o_ref, s_ref = _oracle(x, qk_l2norm=True)
    _check(x, host(o), host(s), o_ref, s_ref)


def test_uniform_channel_gates_match_the_head_gate_path():
    """The same gate on every key channel through the channel-gate kernel equals the
    one-gate-per-head call (the matrix-core path at bf16 d128)."""
    _say("uniform channel gates vs head gate")
    x = make_case(B=1, T=200, Hqk=2, Hv=4, Dk=128, dtype="bf16", g_scale=0.1, init_std=0.02,
                  seed=24, name="uniform")
    d = to_inputs(x)
    gc = d["g"][..., None].expand(-1, -1, -1, x.Dk).contiguous()
    o1, s1 = dn.chunk_fwd(d["q"], d["k"], d["v"], d["beta"], d["g"], d["init"])
    o2, s2 = dn.chunk_fwd(d["q"], d["k"], d["v"], d["beta"], gc, d["init"])
    torch.cuda.synchronize()
    o_ref, s_ref = run_oracle(x)
    _check(x, host(o1), host(s1), o_ref, s_ref)
    _check(x, host(o2), host(s2), o_ref, s_ref)


@pytest.mark.parametrize("Dk,Dv,dtype,norm", [(128, 128, "bf16", False), (64, 32, "f32", False),
                                              (16, 64, "f32", False), (128, 128, "bf16", True)])
def test_decode_channel_gates(Dk, Dv, dtype, norm):
    _say(f"channel gates decode {Dk}x{Dv} {dtype} norm={norm}")
    x = make_case(B=6, T=1, Hqk=2, Hv=4, Dk=Dk, Dv=Dv, dtype=dtype, g_scale=0.3, init_std=0.5,
                  seed=25, decode=True, name=f"decode{Dk}x{Dv}{dtype}", g_per_key=True,
                  qk_raw=norm)
    d = to_inputs(x)
    state = d["init"].clone()
    o = dn.decode_step(d["q"][:, 0], d["k"][:, 0], d["v"][:, 0], d["beta"][:, 0],
                       d["g"][:, 0].contiguous(), state, scale=0.5, qk_l2norm=norm)
    torch.cuda.synchronize()
    o_ref, s_ref = _oracle(x, 0.5, qk_l2norm=norm)
    _check(x, host(o)[:, None], host(state), o_ref, s_ref)


def test_channel_gates_prefill_equals_decode_steps():
    _say("channel gates: prefill vs decode steps")
    x = make_case(B=2, T=40, Hqk=2, Hv=2, Dk=128, dtype="bf16", g_scale=0.1, init_std=0.02,
                  seed=26, name="steps", g_per_key=True)
    d = to_inputs(x)
    o, s = dn.chunk_fwd(d["q"], d["k"], d["v"], d["beta"], d["g"], d["init"])
    state = d["init"].clone()
    outs = []
    for t in range(x.T):
        outs.append(dn.decode_step(d["q"][:, t].contiguous(), d["k"][:, t].contiguous(),
                                   d["v"][:, t].contiguous(), d["beta"][:, t].contiguous(),
                                   d["g"][:, t].contiguous(), state))
    torch.cuda.synchronize()
    od = np.stack([host(t) for t in outs], axis=1)
    o_ref, s_ref = _oracle(x)
    _check(x, od, host(state), o_ref, s_ref)
    _check(x, host(o), host(s), o_ref, s_ref)


def test_decode_channel_gates_full_size():
    """The decode workload (256 sequences x 32 heads, d128 bf16, state ~ N(0, 0.02^2) in
    place) with a log decay per key channel."""
    _say("channel gates decode 256 x 32 heads")
    x = make_case(B=256, T=1, Hqk=32, Dk=128, dtype="bf16", g_scale=0.1, init_std=0.02, seed=0,
                  decode=True, name="decode_full_chg", g_per_key=True)
    d = to_inputs(x)
    state = d["init"].clone()
    o = dn.decode_step(d["q"][:, 0], d["k"][:, 0], d["v"][:, 0], d["beta"][:, 0],
                       d["g"][:, 0].contiguous(), state)
    torch.cuda.synchronize()
    o_ref, s_ref = _oracle(x)
    _check(x, host(o)[:, None], host(state), o_ref, s_ref)


def test_prefill_channel_gates_packed_workload_sample():
    """Packed sequences with initial states and beta in (0, 2), as the 32K-token packed
    workload has them, at 4 sequences of 1,900 tokens in all (the matrix-core kernel)."""
    _say("channel gates packed sample")
    x = make_case(B=1, Hqk=4, Hv=4, Dk=128, dtype="bf16", seqlens=[700, 1, 0, 1199],
                  g_scale=0.05, init_std=0.02, beta_scale=2.0, seed=27, name="packed_chg",
                  g_per_key=True)
    d = to_inputs(x)
    o, s = dn.chunk_fwd(d["q"], d["k"], d["v"], d["beta"], d["g"], d["init"], cu_seqlens=d["cu"])
    torch.cuda.synchronize()
    o_ref, s_ref = _oracle(x)
    _check(x, host(o), host(s), o_ref, s_ref)


@pytest.mark.parametrize("chunk", [32, 64])
def test_channel_gates_bf16_d128_chunk_choice(chunk):
    """bf16 d128 at the default 64-token chunk takes the matrix-core kernel, at 32 the
    vector-ALU one; both agree with the oracle."""
    _say(f"channel gates bf16 d128 chunk {chunk}")
    x = make_case(B=1, T=230, Hqk=2, Hv=2, Dk=128, dtype="bf16", g_scale=0.3, init_std=0.1,
                  seed=28, name=f"bf16chunk{chunk}", g_per_key=True)
    d = to_inputs(x)
    o, s = dn.chunk_fwd(d["q"], d["k"], d["v"], d["beta"], d["g"], d["init"], chunk_size=chunk)
    torch.cuda.synchronize()
    o_ref, s_ref = _oracle(x)
    _check(x, host(o), host(s), o_ref, s_ref)


def test_prefill_channel_gates_layer_workload():
    """The layer-prefill workload (B4 H16 T2048 d128 bf16) with a log decay per key channel
    and an initial state, in the launch configuration the benchmark times: every output and
    final state against the oracle."""
    _say("channel gates prefill B4 H16 T2048")
    x = make_case(B=4, T=2048, Hqk=16, Dk=128, dtype="bf16", g_scale=0.1, init_std=0.02,
                  seed=0, name="layer_chg", g_per_key=True)
    d = to_inputs(x)
    o, s = dn.chunk_fwd(d["q"], d["k"], d["v"], d["beta"], d["g"], d["init"])
    torch.cuda.synchronize()
    o_ref, s_ref = _oracle(x)
    _check(x, host(o), host(s), o_ref, s_ref)


def test_prefill_channel_gates_chunk_edges():
    """Sequence lengths at and around the 64-token chunk and 16-token block edges, empty
    sequences between them, four value heads per q/k head (matrix-core kernel)."""
    _say("channel gates prefill: chunk edges")
    x = make_case(B=1, Hqk=1, Hv=4, Dk=128, dtype="bf16", seqlens=[1, 63, 0, 64, 65, 16, 17, 128, 0],
                  g_scale=0.3, init_std=0.1, beta_scale=2.0, seed=29, name="chg_edges",
                  g_per_key=True)
    d = to_inputs(x)
    o, s = dn.chunk_fwd(d["q"], d["k"], d["v"], d["beta"], d["g"], d["init"], cu_seqlens=d["cu"])
    torch.cuda.synchronize()
    o_ref, s_ref = _oracle(x)
    _check(x, host(o), host(s), o_ref, s_ref)


def test_prefill_channel_gates_graph_replay():
    """The matrix-core channel-gate prefill captured in a HIP graph replays to the eager
    result, every replay, with eager work and synchronisations between the replays."""
    _say("channel gates prefill: graph replay")
    x = make_case(B=2, T=150, Hqk=2, Hv=2, Dk=128, dtype="bf16", g_scale=0.2, init_std=0.05,
                  seed=30, name="chg_graph", g_per_key=True)
    d = to_inputs(x)
    o = torch.empty((2, 150, 2, 128), dtype=torch.bfloat16, device="cuda")
    fs = torch.empty((2, 2, 128, 128), dtype=torch.float32, device="cuda")

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
    o_ref, s_ref = _oracle(x)
    _check(x, host(o), host(fs), o_ref, s_ref)


def test_prefill_channel_gates_without_workspace():
    """With less workspace than the query returns, the matrix-core path runs as one kernel
    (operands formed inside the chunk loop); both forms agree with the oracle and with each
    other bit for bit."""
    _say("channel gates prefill: one kernel vs two")
    x = make_case(B=1, Hqk=2, Hv=4, Dk=128, dtype="bf16", seqlens=[130, 0, 64, 1, 200],
                  g_scale=0.3, init_std=0.1, seed=31, name="chg_nows", g_per_key=True)
    d = to_inputs(x)
    need = dn.workspace_bytes(1, x.T, 2, 4, 128, 128, torch.bfloat16, num_seqs=5, g_per_key=True)
    assert need > 0
    small = torch.empty(16, dtype=torch.uint8, device="cuda")
    o1, s1 = dn.chunk_fwd(d["q"], d["k"], d["v"], d["beta"], d["g"], d["init"], cu_seqlens=d["cu"],
                          workspace=small)
    o2, s2 = dn.chunk_fwd(d["q"], d["k"], d["v"], d["beta"], d["g"], d["init"], cu_seqlens=d["cu"])
    torch.cuda.synchronize()
    o_ref, s_ref = _oracle(x)
    _check(x, host(o1), host(s1), o_ref, s_ref)
    _check(x, host(o2), host(s2), o_ref, s_ref)
    # the same arithmetic in the same order: the two forms agree bit for bit
    assert torch.equal(o1, o2) and torch.equal(s1, s2)


def test_prefill_channel_gates_many_short_sequences():
    """300 packed sequences of 0 to 150 tokens: the per-chunk records are numbered from each
    sequence's start offset (with unused numbers between sequences) and found again by a
    search over the sequence starts; every output and final state against the oracle."""
    _say("channel gates prefill: 300 short sequences")
    rng = np.random.default_rng(32)
    lens = [int(v) for v in rng.integers(0, 151, size=300)]
    x = make_case(B=1, Hqk=1, Hv=2, Dk=128, dtype="bf16", seqlens=lens, g_scale=0.2,
                  init_std=0.1, seed=32, name="chg_many", g_per_key=True)
    d = to_inputs(x)
    o, s = dn.chunk_fwd(d["q"], d["k"], d["v"], d["beta"], d["g"], d["init"], cu_seqlens=d["cu"])
    torch.cuda.synchronize()
    o_ref, s_ref = _oracle(x)
    _check(x, host(o), host(s), o_ref, s_ref)
