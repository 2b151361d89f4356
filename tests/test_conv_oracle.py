"""Pins of the causal-convolution reference (oracle/conv.py): identity and shift filters
(the shift SSM the mutichung page says the convolution generalises), the impulse
response, numpy.convolve per channel, state continuation across a split (CPU only)."""
import numpy as np
import pytest

from oracle.conv import causal_conv


def _x(rng, T, C, B=1):
    return rng.standard_normal((B, T, C))


def test_identity_and_shift_filters():
    rng = np.random.default_rng(1)
    W, C, T = 4, 5, 11
    x = _x(rng, T, C)
    init = rng.standard_normal((1, C, W - 1))
    e_last = np.zeros((C, W)); e_last[:, -1] = 1.0
    y, fin = causal_conv(x, e_last, init_state=init, activation=False)
    np.testing.assert_allclose(y, x, rtol=0, atol=0)
    np.testing.assert_allclose(fin[0], x[0, -(W - 1):].T)
    e_first = np.zeros((C, W)); e_first[:, 0] = 1.0          # a delay of W - 1 tokens
    y, _ = causal_conv(x, e_first, init_state=init, activation=False)
    np.testing.assert_allclose(y[0, W - 1:], x[0, :T - W + 1])
    np.testing.assert_allclose(y[0, :W - 1], init[0].T)


def test_impulse_response_is_the_reversed_filter():
    rng = np.random.default_rng(2)
    W, C, T, t0 = 4, 3, 12, 5
    w = rng.standard_normal((C, W))
    x = np.zeros((1, T, C)); x[0, t0] = 1.0
    y, _ = causal_conv(x, w, activation=False)
    for t in range(T):
        want = w[:, W - 1 - (t - t0)] if 0 <= t - t0 < W else np.zeros(C)
        np.testing.assert_allclose(y[0, t], want, rtol=0, atol=1e-15)


def test_matches_numpy_convolve_with_bias_and_silu():
    rng = np.random.default_rng(3)
    W, C, T = 4, 6, 20
    x, w, b = _x(rng, T, C), rng.standard_normal((C, W)), rng.standard_normal(C)
    y, _ = causal_conv(x, w, b)
    for c in range(C):
        lin = np.convolve(x[0, :, c], w[c, ::-1])[:T] + b[c]
        np.testing.assert_allclose(y[0, :, c], lin / (1 + np.exp(-lin)), rtol=1e-13, atol=1e-14)


def test_split_continues_through_the_state_and_packing_equals_separate_calls():
    rng = np.random.default_rng(4)
    W, C = 4, 5
    lens = [9, 0, 2, 13]
    T = sum(lens)
    cu = np.concatenate([[0], np.cumsum(lens)])
    x, w = _x(rng, T, C), rng.standard_normal((C, W))
    init = rng.standard_normal((len(lens), C, W - 1))
    y, fin = causal_conv(x, w, None, cu, init)
    for n in range(len(lens)):
        a, b = cu[n], cu[n + 1]
        ys, fs = causal_conv(x[:, a:b], w, None, None, init[n:n + 1])
        np.testing.assert_allclose(y[:, a:b], ys, rtol=1e-15)
        np.testing.assert_allclose(fin[n], fs[0], rtol=1e-15)
        if b - a > 3:                       # split one sequence in two through its state
            y1, f1 = causal_conv(x[:, a:a + 3], w, None, None, init[n:n + 1])
            y2, f2 = causal_conv(x[:, a + 3:b], w, None, None, f1)
            np.testing.assert_allclose(np.concatenate([y1, y2], axis=1), ys, rtol=1e-15)
            np.testing.assert_allclose(f2, fs, rtol=1e-15)
    np.testing.assert_allclose(fin[1], init[1])             # empty sequence keeps its state
    np.testing.assert_allclose(fin[2][:, :1], init[2][:, 2:])  # shorter than W - 1: shifted state


def test_bad_offsets():
    with pytest.raises(ValueError):
        causal_conv(np.zeros((1, 5, 2)), np.zeros((2, 4)), cu_seqlens=np.array([0, 3]))


# ------------------------------------------------ the fused prologue (conv_qkv)

def test_conv_qkv_worked_example():
    """One q head (3, 4), one k head (0, 2), one v channel, identity filters, no activation:
    with eps = 0 the heads become (0.6, 0.8) and (0, 1); with eps = 11 the q head is
    (3, 4) / 6 (|u|^2 + eps = 36); v passes through."""
    from oracle.conv import conv_qkv
    x = np.array([[[3.0, 4.0, 0.0, 2.0, -7.0]]])          # [B=1, T=1, C=5]
    w = np.zeros((5, 2)); w[:, -1] = 1.0                    # y_t = x_t
    q, k, v, fin = conv_qkv(x, w, None, 1, 1, 2, 1, activation=False, eps=0.0)
    np.testing.assert_allclose(q[0, 0, 0], [0.6, 0.8], rtol=0, atol=1e-15)
    np.testing.assert_allclose(k[0, 0, 0], [0.0, 1.0], rtol=0, atol=1e-15)
    np.testing.assert_allclose(v[0, 0, 0], [-7.0], rtol=0, atol=0)
    np.testing.assert_allclose(fin[0, :, 0], [3.0, 4.0, 0.0, 2.0, -7.0])
    q, _, _, _ = conv_qkv(x, w, None, 1, 1, 2, 1, activation=False, eps=11.0)
    np.testing.assert_allclose(q[0, 0, 0], [0.5, 4.0 / 6.0], rtol=0, atol=1e-15)


def test_conv_qkv_heads_are_unit_vectors_along_the_conv_output():
    """Against causal_conv on packed sequences with states, bias and silu, GQA heads: every
    q and k head is parallel to the convolution's head (cosine 1) with norm
    |u| / sqrt(|u|^2 + eps); v and the final state are the convolution's, exactly; without
    the norm all three are the convolution's channels in order."""
    from oracle.conv import conv_qkv
    rng = np.random.default_rng(5)
    Hqk, Hv, Dk, Dv, W = 2, 4, 8, 4, 4
    C = 2 * Hqk * Dk + Hv * Dv
    lens = [7, 0, 1, 12]
    T = sum(lens)
    cu = np.concatenate([[0], np.cumsum(lens)])
    x, w, b = _x(rng, T, C), rng.standard_normal((C, W)), rng.standard_normal(C)
    init = rng.standard_normal((len(lens), C, W - 1))
    eps = 0.3
    u, fin_ref = causal_conv(x, w, b, cu, init)
    q, k, v, fin = conv_qkv(x, w, b, Hqk, Hv, Dk, Dv, cu, init, eps=eps)
    np.testing.assert_array_equal(fin, fin_ref)
    np.testing.assert_array_equal(v.reshape(1, T, Hv * Dv), u[..., 2 * Hqk * Dk:])
    for got, lo in ((q, 0), (k, Hqk * Dk)):
        uh = u[..., lo:lo + Hqk * Dk].reshape(1, T, Hqk, Dk)
        nu = np.linalg.norm(uh, axis=-1)
        np.testing.assert_allclose(np.linalg.norm(got, axis=-1), nu / np.sqrt(nu ** 2 + eps), rtol=1e-13)
        cos = np.sum(got * uh, axis=-1) / (np.linalg.norm(got, axis=-1) * nu)
        np.testing.assert_allclose(cos, 1.0, rtol=1e-13)
    q0, k0, v0, _ = conv_qkv(x, w, b, Hqk, Hv, Dk, Dv, cu, init, qk_l2norm=False)
    np.testing.assert_array_equal(np.concatenate([q0.reshape(1, T, -1), k0.reshape(1, T, -1),
                                                  v0.reshape(1, T, -1)], axis=-1), u)


def test_conv_qkv_rejects_a_split_that_does_not_add_up():
    from oracle.conv import conv_qkv
    x = np.zeros((1, 3, 10))
    with pytest.raises(ValueError):
        conv_qkv(x, np.ones((10, 2)), None, 1, 1, 4, 4)
