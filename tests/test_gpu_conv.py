"""The short causal depthwise convolution (+ silu) on the HIP path against the fp64
reference oracle/conv.py (needs an MI355X): prompts with packed sequences and conv states,
and the decode step with its state updated in place.

Bar: relative L2 over the whole tensor, 1e-4 for fp32, 1e-2 for bf16; conv states hold
copies of inputs and must match bit for bit.
"""
import sys

import numpy as np
import pytest
import torch

import delta_rule_recurrent_chunked_amd as dn
from oracle.conv import causal_conv as ref_conv
from synth import f32_to_bf16_bits, to_f64
from tests.gpu_util import dev_tensor, host, rel_l2

pytestmark = pytest.mark.gpu


def _say(*a):
    print(*a, flush=True)
    sys.stdout.flush()


def _cast(a, dtype):
    a = a.astype(np.float32)
    return f32_to_bf16_bits(a) if dtype == "bf16" else a


def _inputs(rng, B, T, C, W, N, dtype):
    x = _cast(rng.standard_normal((B, T, C)), dtype)
    w = (rng.standard_normal((C, W)) / np.sqrt(W)).astype(np.float32)
    b = (0.1 * rng.standard_normal(C)).astype(np.float32)
    s0 = _cast(rng.standard_normal((N, C, W - 1)), dtype)
    return x, w, b, s0


@pytest.mark.parametrize("dtype", ["f32", "bf16"])
@pytest.mark.parametrize("W", [2, 4, 8])
def test_conv_packed_sequences(dtype, W):
    _say(f"causal conv packed W={W} {dtype}")
    rng = np.random.default_rng(W)
    lens = [0, 5, 1, 40, 77, 0, 33]          # crosses 32-token blocks, empty sequences
    T, C, N = sum(lens), 48, len(lens)
    cu = np.concatenate([[0], np.cumsum(lens)]).astype(np.int32)
    x, w, b, s0 = _inputs(rng, 1, T, C, W, N, dtype)
    y, sT = dn.causal_conv(dev_tensor(x), dev_tensor(w), dev_tensor(b), dev_tensor(s0),
                           cu_seqlens=dev_tensor(cu))
    torch.cuda.synchronize()
    y_ref, s_ref = ref_conv(to_f64(x), w, b, cu, to_f64(s0))
    err = rel_l2(host(y), y_ref)
    _say(f"  rel_l2 y={err:.2e}")
    assert err <= (1e-4 if dtype == "f32" else 1e-2)
    assert np.array_equal(host(sT), s_ref)


def test_conv_batch_rows_without_state_bias_or_activation():
    _say("causal conv batch rows, plain")
    rng = np.random.default_rng(5)
    x, w, _, _ = _inputs(rng, 3, 70, 64, 4, 3, "f32")
    y, sT = dn.causal_conv(dev_tensor(x), dev_tensor(w), activation=None)
    torch.cuda.synchronize()
    y_ref, s_ref = ref_conv(x, w, activation=False)
    assert rel_l2(host(y), y_ref) <= 1e-5
    assert np.array_equal(host(sT), s_ref)


def test_conv_steps_equal_the_prompt_call():
    """T decode steps from a conv state equal one prompt call over the T tokens."""
    _say("causal conv steps vs prompt")
    rng = np.random.default_rng(6)
    N, T, C, W = 5, 9, 64, 4
    x, w, b, s0 = _inputs(rng, N, T, C, W, N, "bf16")
    xd = dev_tensor(x)
    st = dev_tensor(s0).clone()
    wd, bd = dev_tensor(w), dev_tensor(b)
    ys = [dn.causal_conv_step(xd[:, t].contiguous(), wd, bd, st) for t in range(T)]
    y, sT = dn.causal_conv(xd, wd, bd, dev_tensor(s0))
    torch.cuda.synchronize()
    y_ref, s_ref = ref_conv(to_f64(x), w, b, None, to_f64(s0))
    assert rel_l2(np.stack([host(t) for t in ys], axis=1), y_ref) <= 1e-2
    assert rel_l2(host(y), y_ref) <= 1e-2
    assert torch.equal(st, sT) and np.array_equal(host(sT), s_ref)


def test_conv_layer_workload():
    """The q, k, v channels of the layer workload (B4 T2048, 16 heads x 128 x 3 = 6144
    channels, bf16, width 4) in one call."""
    _say("causal conv B4 T2048 C6144")
    rng = np.random.default_rng(7)
    x, w, b, _ = _inputs(rng, 4, 2048, 6144, 4, 4, "bf16")
    y, sT = dn.causal_conv(dev_tensor(x), dev_tensor(w), dev_tensor(b))
    torch.cuda.synchronize()
    y_ref, s_ref = ref_conv(to_f64(x), w, b)
    err = rel_l2(host(y), y_ref)
    _say(f"  rel_l2 y={err:.2e}")
    assert err <= 1e-2 and np.array_equal(host(sT), s_ref)


# ------------------------------------------- the fused prologue (dn_conv_qkv)

def _qkv_check(x, w, b, s0, cu, heads, dtype, norm=True, eps=1e-6):
    Hqk, Hv, Dk, Dv = heads
    from oracle.conv import conv_qkv as ref_qkv
    q, k, v, sT = dn.conv_qkv(dev_tensor(x), dev_tensor(w), None if b is None else dev_tensor(b),
                              Hqk, Hv, Dk, Dv,
                              initial_state=None if s0 is None else dev_tensor(s0),
                              cu_seqlens=None if cu is None else dev_tensor(cu), qk_l2norm=norm, eps=eps)
    torch.cuda.synchronize()
    rq, rk, rv, rs = ref_qkv(to_f64(x) if dtype == "bf16" else x, w, b, Hqk, Hv, Dk, Dv, cu,
                             None if s0 is None else (to_f64(s0) if dtype == "bf16" else s0),
                             qk_l2norm=norm, eps=eps)
    bar = 1e-4 if dtype == "f32" else 1e-2
    errs = {n: rel_l2(host(a), r) for n, a, r in (("q", q, rq), ("k", k, rk), ("v", v, rv))}
    # every q / k head of every token against its own norm (a wrong head fails it)
    worst = 0.0
    for a, r in ((q, rq), (k, rk)):
        d = np.linalg.norm((host(a).astype(np.float64) - r).reshape(-1, Dk), axis=-1)
        n = np.maximum(np.linalg.norm(r.reshape(-1, Dk), axis=-1), 1e-3)
        worst = max(worst, float(np.max(d / n)))
    _say(f"  rel_l2 q={errs['q']:.2e} k={errs['k']:.2e} v={errs['v']:.2e}; worst head {worst:.2e} (bar {bar:.0e})")
    assert max(errs.values()) <= bar and worst <= (3 * bar if dtype == "bf16" else bar)
    assert np.array_equal(host(sT), rs)


@pytest.mark.parametrize("dtype", ["f32", "bf16"])
@pytest.mark.parametrize("heads", [(2, 4, 128, 128), (1, 1, 64, 32), (3, 3, 32, 16), (1, 2, 16, 8)],
                         ids=["gqa_d128", "d64", "d32_odd_heads", "d16"])
def test_conv_qkv_packed(dtype, heads):
    """dn_conv_qkv on packed sequences (empty ones, a block-crossing mix) with conv states:
    q, k, v and the final state against oracle/conv.py's conv_qkv; channel counts that end
    inside a wave and q/k heads of 2 to 16 lanes."""
    Hqk, Hv, Dk, Dv = heads
    C = 2 * Hqk * Dk + Hv * Dv
    _say(f"conv_qkv packed heads={heads} C={C} {dtype}")
    rng = np.random.default_rng(C)
    lens = [0, 5, 1, 70, 130, 0, 33]
    T, N = sum(lens), len(lens)
    cu = np.concatenate([[0], np.cumsum(lens)]).astype(np.int32)
    x, w, b, s0 = _inputs(rng, 1, T, C, 4, N, dtype)
    _qkv_check(x, w, b, s0, cu, heads, dtype)


def test_conv_qkv_rows_without_norm_or_state():
    """Batch rows, no state, no L2 norm: the three outputs are the convolution's channels."""
    _say("conv_qkv rows, no norm")
    rng = np.random.default_rng(9)
    heads = (2, 2, 64, 64)
    x, w, b, _ = _inputs(rng, 3, 100, 2 * 2 * 64 + 2 * 64, 3, 3, "bf16")
    _qkv_check(x, w, b, None, None, heads, "bf16", norm=False)


def test_conv_qkv_layer_workload_then_rule():
    """The layer workload (B4 T2048, 16 heads, d128, bf16, width 4): the prologue against
    the oracle, then its q, k, v through dn_chunk_fwd agree with dn_chunk_fwd normalising
    the plain convolution's q, k inside the call."""
    _say("conv_qkv B4 T2048 H16 d128 + chunk_fwd")
    rng = np.random.default_rng(10)
    H, D = 16, 128
    x, w, b, _ = _inputs(rng, 4, 2048, 3 * H * D, 4, 4, "bf16")
    _qkv_check(x, w, b, None, None, (H, H, D, D), "bf16")
    xd, wd, bd = dev_tensor(x), dev_tensor(w), dev_tensor(b)
    q, k, v, _ = dn.conv_qkv(xd, wd, bd, H, H, D, D)
    y, _ = dn.causal_conv(xd, wd, bd)
    beta = torch.sigmoid(torch.randn((4, 2048, H), device="cuda"))
    o1, s1 = dn.chunk_fwd(q, k, v, beta, None, None)
    yq = y[..., :H * D].reshape(4, 2048, H, D).contiguous()
    yk = y[..., H * D:2 * H * D].reshape(4, 2048, H, D).contiguous()
    yv = y[..., 2 * H * D:].reshape(4, 2048, H, D).contiguous()
    o2, s2 = dn.chunk_fwd(yq, yk, yv, beta, None, None, qk_l2norm=True)
    torch.cuda.synchronize()
    eo, es = rel_l2(host(o1), host(o2)), rel_l2(host(s1), host(s2))
    _say(f"  prologue + rule vs rule normalising: o {eo:.2e} state {es:.2e}")
    assert eo <= 1e-2 and es <= 1e-2
