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
