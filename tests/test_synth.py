"""The seeded input generator: determinism, shapes, ranges and the bf16 cast."""
import numpy as np
import pytest
import torch

from synth import make_case, make_config, f32_to_bf16_bits, bf16_bits_to_f32


def test_deterministic_per_seed():
    a = make_case(B=2, T=33, Hqk=2, Hv=4, Dk=8, Dv=16, dtype="bf16", g_scale=0.1,
                  init_std=0.02, seed=5)
    b = make_case(B=2, T=33, Hqk=2, Hv=4, Dk=8, Dv=16, dtype="bf16", g_scale=0.1,
                  init_std=0.02, seed=5)
    c = make_case(B=2, T=33, Hqk=2, Hv=4, Dk=8, Dv=16, dtype="bf16", g_scale=0.1,
                  init_std=0.02, seed=6)
    for name in ("q", "k", "v", "beta", "g", "init"):
        assert np.array_equal(getattr(a, name), getattr(b, name))
    assert not np.array_equal(a.q, c.q)


def test_shapes_and_ranges():
    x = make_case(B=3, T=50, Hqk=2, Hv=6, Dk=16, Dv=32, dtype="f32", beta_scale=2.0,
                  g_scale=0.05, init_std=0.02, seed=1)
    assert x.q.shape == (3, 50, 2, 16) and x.k.shape == (3, 50, 2, 16)
    assert x.v.shape == (3, 50, 6, 32)
    assert x.beta.shape == (3, 50, 6) and x.beta.dtype == np.float32
    assert x.g.shape == (3, 50, 6) and x.g.dtype == np.float32
    assert x.init.shape == (3, 6, 16, 32)
    assert np.all((x.beta > 0) & (x.beta < 2)) and np.any(x.beta > 1)
    assert np.all(x.g <= 0)
    # q and k are unit vectors per (token, head)
    np.testing.assert_allclose(np.linalg.norm(x.q, axis=-1), 1.0, rtol=1e-6)
    np.testing.assert_allclose(np.linalg.norm(x.k, axis=-1), 1.0, rtol=1e-6)


def test_bf16_round_to_nearest_even_matches_torch():
    rng = np.random.default_rng(0)
    x = np.concatenate([rng.standard_normal(100000).astype(np.float32),
                        np.array([1.00390625, 1.01171875, -1.00390625, 0.0, -0.0], np.float32)])
    bits = f32_to_bf16_bits(x)
    ref = torch.from_numpy(x).to(torch.bfloat16).view(torch.int16).numpy().view(np.uint16)
    assert np.array_equal(bits, ref)
    back = bf16_bits_to_f32(bits)
    assert np.array_equal(back, torch.from_numpy(x).to(torch.bfloat16).float().numpy())


def test_packed_cuts():
    x = make_case(B=1, T=1000, Hqk=2, Dk=8, dtype="bf16", num_seqs_cut=8, seed=3)
    cu = x.cu_seqlens
    assert cu.dtype == np.int32 and len(cu) == 9
    assert cu[0] == 0 and cu[-1] == 1000 and np.all(np.diff(cu) > 0)
    y = make_case(B=1, Hqk=2, Dk=8, seqlens=[5, 0, 7], seed=3)
    assert list(y.cu_seqlens) == [0, 5, 5, 12] and y.T == 12


@pytest.mark.parametrize("i", [1, 4])
def test_small_configs(i):
    x = make_config(i)
    if i == 1:
        assert (x.B, x.T, x.Hqk, x.Hv, x.Dk, x.Dv, x.dtype) == (1, 64, 2, 2, 16, 16, "f32")
        assert x.g is None and x.init is None
    else:
        assert x.decode and (x.B, x.T, x.Hv, x.Dk) == (256, 1, 32, 128)
        assert x.init.shape == (256, 32, 128, 128)
        assert abs(float(x.init.std()) - 0.02) < 1e-3
