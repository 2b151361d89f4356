"""The chunkwise reverse pass (dn_chunk_bwd) against the fp64 reverse-pass reference
oracle/backward.py (needs an MI355X).

Bar: relative L2 1e-2 (bf16 inputs) on every gradient over the whole tensor, and for every
(sequence, head) the unit's error against the larger of its own norm and its share of the
tensor's norm (|ref| sqrt(unit size / tensor size)): a unit computed wrong fails it, while a
one-token unit whose gradient happens to be small (dg of a lone token, a difference of
terms each rounded through bf16 operands) is held to the tensor's scale.
"""
import sys

import numpy as np
import pytest
import torch

import delta_rule_recurrent_chunked_amd as dn
from oracle.backward import backward as ref_backward
from synth import f32_to_bf16_bits, make_case
from tests.gpu_util import dev_tensor, host, log_errors, rel_l2, to_inputs, tol

pytestmark = pytest.mark.gpu


def _say(*a):
    print(*a, flush=True)
    sys.stdout.flush()


def _run(x, scale=1.0, seed=81, qk_l2norm=False):
    rng = np.random.default_rng(seed)
    N = x.num_seqs
    do_dev = dev_tensor(f32_to_bf16_bits(rng.standard_normal((x.B, x.T, x.Hv, x.Dv)).astype(np.float32)))
    dfin = (0.1 * rng.standard_normal((N, x.Hv, x.Dk, x.Dv))).astype(np.float32)
    d = to_inputs(x)
    grads = dn.chunk_bwd(d["q"], d["k"], d["v"], d["beta"], d["g"], d["init"], do_dev,
                         dev_tensor(dfin), cu_seqlens=d["cu"], scale=scale, qk_l2norm=qk_l2norm)
    torch.cuda.synchronize()
    return grads, host(do_dev), dfin.astype(np.float64), d, do_dev


def _check(x, grads, do, dfin, scale=1.0, qk_l2norm=False):
    f = x.f64()
    ref = ref_backward(f["q"], f["k"], f["v"], f["beta"], f["g"], f["init"], do, dfin,
                       x.cu_seqlens, scale, qk_l2norm=qk_l2norm)
    bounds = x.seq_bounds()
    errs = {}
    pairs = [("dq", "dq"), ("dk", "dk"), ("dv", "dv"), ("dbeta", "dbeta"),
             ("d_initial_state", "dinit")] + ([("dg", "dg")] if x.g is not None else [])
    for got, want in pairs:
        a, b = host(grads[got]), ref[want]
        err = rel_l2(a, b)
        worst = 0.0
        total = np.linalg.norm(b.ravel())

        def unit(au, bu):
            scale_u = max(np.linalg.norm(bu.ravel()), total * np.sqrt(bu.size / b.size))
            return float(np.linalg.norm((au - bu).ravel()) / scale_u) if scale_u > 0 else 0.0

        if got == "d_initial_state":
            for n in range(a.shape[0]):
                for h in range(a.shape[1]):
                    worst = max(worst, unit(a[n, h], b[n, h]))
        else:   # per (sequence, head) over the sequence's tokens
            af, bf = a.reshape((x.B * x.T, a.shape[2]) + a.shape[3:]), b.reshape((x.B * x.T, b.shape[2]) + b.shape[3:])
            for n in range(len(bounds) - 1):
                s, e = int(bounds[n]), int(bounds[n + 1])
                if e > s:
                    for h in range(af.shape[1]):
                        worst = max(worst, unit(af[s:e, h], bf[s:e, h]))
        errs[got] = err
        errs["worst_" + got] = worst
        _say(f"  {got}: rel_l2 {err:.2e}, worst (sequence, head) {worst:.2e}")
        assert np.all(np.isfinite(a)), got
        assert err <= tol(x) and worst <= tol(x), got
    log_errors(x.name, bar=tol(x), **errs)


CASES = {
    "gated_ragged_init": dict(B=2, T=200, Hqk=2, Hv=2, Dk=128, g_scale=0.1, init_std=0.02,
                              beta_scale=2.0),
    "plain_rows": dict(B=2, T=130, Hqk=2, Hv=2, Dk=128),
    "gated_packed_gqa": dict(B=1, Hqk=1, Hv=2, Dk=128, seqlens=[70, 0, 1, 129, 64], g_scale=0.3,
                             init_std=0.02, beta_scale=2.0),
    "strong_decay": dict(B=1, T=300, Hqk=2, Hv=4, Dk=128, g_scale=3.0, init_std=0.02),
    # at least one states workgroup per CU (sequences x value heads x 4 slices >= 256): the
    # states launch writes the T^T and P records itself and nothing runs beside it
    "full_chip_gated_ragged": dict(B=2, T=200, Hqk=8, Hv=32, Dk=128, g_scale=0.1, init_std=0.02,
                                   beta_scale=2.0),
    "full_chip_plain_rows": dict(B=4, T=130, Hqk=16, Hv=16, Dk=128),
    "full_chip_packed_strong_decay": dict(B=1, Hqk=8, Hv=16, Dk=128, seqlens=[70, 0, 1, 129, 64, 300],
                                          g_scale=3.0, init_std=0.02),
}


@pytest.mark.parametrize("name", sorted(CASES))
def test_chunk_bwd(name):
    _say(f"chunk bwd {name}")
    x = make_case(dtype="bf16", seed=80, name=f"chunk_bwd_{name}", **CASES[name])
    grads, do, dfin, _, _ = _run(x, scale=0.8)
    _check(x, grads, do, dfin, scale=0.8)


NORM_CASES = {
    "norm_gated_ragged": dict(B=2, T=200, Hqk=2, Hv=2, Dk=128, g_scale=0.1, init_std=0.02),
    "norm_packed_gqa": dict(B=1, Hqk=1, Hv=2, Dk=128, seqlens=[70, 0, 1, 129, 64], g_scale=0.3,
                            init_std=0.02, beta_scale=2.0),
    "norm_plain": dict(B=1, T=130, Hqk=2, Hv=2, Dk=128),
    "norm_full_chip_gated": dict(B=2, T=150, Hqk=16, Hv=32, Dk=128, g_scale=0.1, init_std=0.02),
}


@pytest.mark.parametrize("name", sorted(NORM_CASES))
def test_chunk_bwd_in_call_normalisation(name):
    """Raw N(0, 1) q and k (norms about sqrt(128)), normalised inside the call: the gradients
    for the raw rows against the fp64 reverse pass through the same normalisation."""
    _say(f"chunk bwd, in-call normalisation, {name}")
    x = make_case(dtype="bf16", seed=88, name=f"chunk_bwd_{name}", qk_raw=True, **NORM_CASES[name])
    grads, do, dfin, _, _ = _run(x, scale=0.9, qk_l2norm=True)
    _check(x, grads, do, dfin, scale=0.9, qk_l2norm=True)


def test_chunk_bwd_layer_workload():
    """B1 H16 T2048 d128 bf16 with one gate per head: every gradient against the fp64
    reverse pass."""
    _say("chunk bwd B1 H16 T2048 gated")
    x = make_case(B=1, T=2048, Hqk=16, Dk=128, dtype="bf16", g_scale=0.1, init_std=0.02, seed=82,
                  name="chunk_bwd_B1_H16_T2048")
    grads, do, dfin, _, _ = _run(x)
    _check(x, grads, do, dfin)


def test_chunk_bwd_layer_workload_b4():
    """B4 H16 T2048 d128 bf16 gated, the reverse-pass shape the benchmark times at B4: 256
    states workgroups, so the states launch writes the T^T and P records and every launch
    runs on the caller's stream."""
    _say("chunk bwd B4 H16 T2048 gated")
    x = make_case(B=4, T=2048, Hqk=16, Dk=128, dtype="bf16", g_scale=0.1, init_std=0.02, seed=89,
                  name="chunk_bwd_B4_H16_T2048")
    grads, do, dfin, _, _ = _run(x)
    _check(x, grads, do, dfin)


def test_chunk_bwd_bitwise_repeatable_and_agrees_with_recurrent():
    """Two calls agree bit for bit; the token-by-token reverse pass (dn_recurrent_bwd, a
    different algorithm on the GPU) agrees with it to the bf16 bar."""
    _say("chunk bwd repeat + recurrent agreement")
    x = make_case(B=1, Hqk=2, Hv=2, Dk=128, dtype="bf16", seqlens=[100, 37], g_scale=0.1,
                  init_std=0.02, seed=83, name="chunk_bwd_repeat")
    g1, _, _, d, do_dev = _run(x)
    g2, _, _, _, _ = _run(x)
    for k in g1:
        if g1[k] is not None:
            assert torch.equal(g1[k], g2[k]), k
    _, _, trace = dn.recurrent_fwd(d["q"], d["k"], d["v"], d["beta"], d["g"], d["init"],
                                   cu_seqlens=d["cu"], state_trace=True)
    rng = np.random.default_rng(81)
    rng.standard_normal((x.B, x.T, x.Hv, x.Dv))
    dfin = dev_tensor((0.1 * rng.standard_normal((x.num_seqs, x.Hv, x.Dk, x.Dv))).astype(np.float32))
    r = dn.recurrent_bwd(d["q"], d["k"], d["v"], d["beta"], d["g"], d["init"], trace, do_dev, dfin,
                         cu_seqlens=d["cu"])
    torch.cuda.synchronize()
    for k in ("dq", "dk", "dv", "dbeta", "dg", "d_initial_state"):
        err = rel_l2(host(g1[k]), host(r[k]))
        _say(f"  {k}: chunked vs token-by-token {err:.2e}")
        assert err <= 1e-2, k


def test_chunk_bwd_rejects_unsupported():
    x = make_case(B=1, T=64, Hqk=1, Dk=64, dtype="bf16", seed=84)
    d = to_inputs(x)
    do = torch.zeros((1, 64, 1, 64), dtype=torch.bfloat16, device="cuda")
    with pytest.raises(NotImplementedError):
        dn.chunk_bwd(d["q"], d["k"], d["v"], d["beta"], None, None, do)


@pytest.mark.parametrize("Hqk,Hv", [(2, 2), (16, 32)])
def test_chunk_bwd_graph_replay(Hqk, Hv):
    """dn_chunk_bwd captured in a HIP graph (with few heads its chunk-start states run on a
    second stream, forked from and joined back to the captured one by events; with 32 heads
    at B2 every launch runs on the captured stream): three replays, each after an eager call
    on other inputs that rewrites the workspace, match the eager result bit for bit."""
    _say(f"chunk bwd graph capture + replays, {Hqk} -> {Hv} heads")
    x = make_case(B=2, T=200, Hqk=Hqk, Hv=Hv, Dk=128, dtype="bf16", g_scale=0.1, init_std=0.02,
                  seed=85, name="chunk_bwd_graph")
    y = make_case(B=2, T=200, Hqk=Hqk, Hv=Hv, Dk=128, dtype="bf16", g_scale=0.2, init_std=0.02,
                  seed=86, name="chunk_bwd_graph_other")
    rng = np.random.default_rng(87)
    do = dev_tensor(f32_to_bf16_bits(rng.standard_normal((2, 200, Hv, 128)).astype(np.float32)))
    d, e = to_inputs(x), to_inputs(y)
    ws = torch.empty(dn.chunk_bwd_workspace_bytes(2, 200, Hqk, Hv, 128, 128, torch.bfloat16),
                     dtype=torch.uint8, device="cuda")
    args = (d["q"], d["k"], d["v"], d["beta"], d["g"], d["init"], do)
    other = (e["q"], e["k"], e["v"], e["beta"], e["g"], e["init"], do)
    eager = dn.chunk_bwd(*args, workspace=ws)
    torch.cuda.synchronize()
    side = torch.cuda.Stream()
    side.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(side):
        dn.chunk_bwd(*args, workspace=ws)
    torch.cuda.current_stream().wait_stream(side)
    torch.cuda.synchronize()
    graph = torch.cuda.CUDAGraph()
    with torch.cuda.graph(graph):
        out = dn.chunk_bwd(*args, workspace=ws)
    for rep in range(3):
        dn.chunk_bwd(*other, workspace=ws)
        torch.cuda.synchronize()
        graph.replay()
        torch.cuda.synchronize()
        for k, v in eager.items():
            if v is not None:
                assert torch.equal(out[k], v), (rep, k)
    _say("  three replays match the eager call")
