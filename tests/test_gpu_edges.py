"""Edges of the method on the matrix-core prompt kernel and the reverse pass, against the
fp64 oracles (needs an MI355X).

* strong decay: one log decay per head with g = -c softplus(z), c = 3 and 5 (a chunk then
  decays by e^-100 and more), plain and normalised in the call;
* in-call normalisation with raw key and query norms spread log-uniformly over 0.05 .. 20,
  and with key norms differing by 10^4 inside every chunk (the limit the header states);
* the reverse pass at the length the benchmark times (T = 2048) on two heads.

Bar: relative L2 1e-2 (bf16 inputs) on the whole tensors and on every (sequence, value head).
"""
import sys

import numpy as np
import pytest
import torch

import delta_rule_recurrent_chunked_amd as dn
from synth import bf16_bits_to_f32, f32_to_bf16_bits, make_case
from tests.gpu_util import dev_tensor, host, log_errors, per_unit_rel, rel_l2, to_inputs, tol

pytestmark = pytest.mark.gpu


def _say(*a):
    print(*a, flush=True)
    sys.stdout.flush()


def _oracle(x, scale=1.0, qk_l2norm=False, eps=1e-6):
    import oracle
    f = x.f64()
    return oracle.recurrent(f["q"], f["k"], f["v"], f["beta"], f["g"], f["init"],
                            x.cu_seqlens, scale=scale, qk_l2norm=qk_l2norm, eps=eps)


def _check(x, o, s, o_ref, s_ref):
    eo, es = rel_l2(o, o_ref), rel_l2(s, s_ref)
    uo, us, where = per_unit_rel(o, o_ref, s, s_ref, x)
    _say(f"  {x.name}: rel_l2 o={eo:.2e} state={es:.2e}; worst (sequence, head) o={uo:.2e} "
         f"state={us:.2e} at {where} (bar {tol(x):.0e})")
    log_errors(x.name, o=eo, state=es, worst_unit_o=uo, worst_unit_state=us, bar=tol(x),
               worst_unit=where)
    assert np.all(np.isfinite(o)) and np.all(np.isfinite(s))
    assert max(eo, es, uo, us) <= tol(x)


def _run(x, scale=1.0, qk_l2norm=False, eps=1e-6):
    assert dn.chunk_fwd_path(x.B, x.T, x.Hqk, x.Hv, x.Dk, x.Dv, torch.bfloat16,
                             num_seqs=x.num_seqs, qk_l2norm=qk_l2norm) == "fused"
    d = to_inputs(x)
    o, s = dn.chunk_fwd(d["q"], d["k"], d["v"], d["beta"], d["g"], d["init"], cu_seqlens=d["cu"],
                        scale=scale, qk_l2norm=qk_l2norm, l2norm_eps=eps)
    torch.cuda.synchronize()
    o_ref, s_ref = _oracle(x, scale, qk_l2norm, eps)
    _check(x, host(o), host(s), o_ref, s_ref)


# ------------------------------------------------------------------------ strong decay

@pytest.mark.parametrize("c", [3.0, 5.0])
@pytest.mark.parametrize("norm", [False, True], ids=["prenormalised", "in_call_norm"])
def test_fused_strong_decay(c, norm):
    _say(f"fused kernel, g = -{c} softplus(z), in-call norm {norm}")
    x = make_case(B=2, T=333, Hqk=2, Hv=4, Dk=128, dtype="bf16", g_scale=c, init_std=0.02,
                  beta_scale=2.0, seed=61, name=f"strong_decay_{c}_{'norm' if norm else 'pre'}",
                  qk_raw=norm)
    _run(x, scale=0.8, qk_l2norm=norm)


def test_fused_strong_decay_packed():
    _say("fused kernel, g = -4 softplus(z), packed sequences")
    x = make_case(B=1, Hqk=2, Hv=4, Dk=128, dtype="bf16", seqlens=[1, 130, 0, 64, 257, 15],
                  g_scale=4.0, init_std=0.02, beta_scale=2.0, seed=62, name="strong_decay_packed")
    _run(x)


# ---------------------------------------------------- in-call normalisation, norm spreads

def _with_norms(x, knorm, qnorm):
    """x with every raw q/k vector rescaled to the given norms ([B, T, Hqk] each), rounded
    to bf16 again (both sides then read the same bits)."""
    for name, nrm in (("k", knorm), ("q", qnorm)):
        a = bf16_bits_to_f32(getattr(x, name)).astype(np.float64)
        a = a / np.linalg.norm(a, axis=-1, keepdims=True) * nrm[..., None]
        setattr(x, name, f32_to_bf16_bits(a.astype(np.float32)))
    return x


def test_in_call_norm_spread_norms():
    """Raw q and k norms drawn log-uniformly over 0.05 .. 20 per token (the spread the CPU
    pins use), gated, packed, GQA."""
    _say("in-call normalisation, norms 0.05 .. 20")
    x = make_case(B=1, Hqk=2, Hv=4, Dk=128, dtype="bf16", seqlens=[200, 1, 129, 64, 0, 333],
                  g_scale=0.1, init_std=0.02, beta_scale=2.0, seed=63, name="norm_spread",
                  qk_raw=True)
    rng = np.random.default_rng(64)
    shape = (x.B, x.T, x.Hqk)
    _with_norms(x, np.exp(rng.uniform(np.log(0.05), np.log(20.0), shape)),
                np.exp(rng.uniform(np.log(0.05), np.log(20.0), shape)))
    _run(x, qk_l2norm=True)


@pytest.mark.parametrize("gated", [False, True])
def test_in_call_norm_key_ratio_1e4(gated):
    """Key norms 10^-2 and 10^2 alternating token by token, so every chunk holds keys whose
    norms differ by 10^4 (query norms alternate the other way)."""
    _say(f"in-call normalisation, key norm ratio 1e4, gated {gated}")
    x = make_case(B=2, T=300, Hqk=2, Hv=2, Dk=128, dtype="bf16", g_scale=0.1 if gated else None,
                  init_std=0.02, seed=65, name=f"norm_ratio_1e4_{'gated' if gated else 'plain'}",
                  qk_raw=True)
    alt = np.where(np.arange(x.T) % 2 == 0, 1e-2, 1e2)
    kn = np.broadcast_to(alt[None, :, None], (x.B, x.T, x.Hqk))
    qn = np.broadcast_to(alt[::-1].copy()[None, :, None], (x.B, x.T, x.Hqk))
    _with_norms(x, kn, qn)
    _run(x, qk_l2norm=True)


# -------------------------------------------------------- reverse pass at T = 2048

def test_reverse_pass_T2048():
    """dn_recurrent_bwd on one gated 2048-token sequence of two heads (the benchmark's
    length), every gradient against oracle/backward.py, whole tensors and per head."""
    from oracle.backward import backward as ref_backward
    _say("reverse pass B1 H2 T2048 d128 bf16 gated")
    x = make_case(B=1, T=2048, Hqk=2, Hv=2, Dk=128, dtype="bf16", g_scale=0.1, init_std=0.02,
                  seed=66, name="bwd_T2048")
    rng = np.random.default_rng(67)
    do_dev = dev_tensor(f32_to_bf16_bits(rng.standard_normal((1, 2048, 2, 128)).astype(np.float32)))
    dfin = rng.standard_normal((1, 2, 128, 128)).astype(np.float32)
    d = to_inputs(x)
    _, _, trace = dn.recurrent_fwd(d["q"], d["k"], d["v"], d["beta"], d["g"], d["init"],
                                   state_trace=True)
    grads = dn.recurrent_bwd(d["q"], d["k"], d["v"], d["beta"], d["g"], d["init"], trace, do_dev,
                             dev_tensor(dfin))
    torch.cuda.synchronize()
    del trace
    f = x.f64()
    ref = ref_backward(f["q"], f["k"], f["v"], f["beta"], f["g"], f["init"], host(do_dev),
                       dfin.astype(np.float64))
    errs = {}
    for got, want in (("dq", "dq"), ("dk", "dk"), ("dv", "dv"), ("dbeta", "dbeta"),
                      ("dg", "dg"), ("d_initial_state", "dinit")):
        a, b = host(grads[got]), ref[want]
        err = rel_l2(a, b)
        per_head = max(rel_l2(a[:, :, h], b[:, :, h]) if a.ndim >= 3 else rel_l2(a[h], b[h])
                       for h in range(2)) if got != "d_initial_state" else \
            max(rel_l2(a[0, h], b[0, h]) for h in range(2))
        errs[got] = err
        _say(f"  {got}: rel_l2 {err:.2e}, worst head {per_head:.2e}")
        assert err <= tol(x) and per_head <= tol(x), got
    log_errors(x.name, bar=tol(x), **errs)
