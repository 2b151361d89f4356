"""The chunkwise algebra the prefill kernels use, checked in fp64 against the oracle."""
import numpy as np
import pytest

import oracle
from synth import make_case, f32_to_bf16_bits, bf16_bits_to_f32
from tests.chunk_model import blocked_unit_lower_inverse, chunked
from tests.conftest import rel_l2


def test_blocked_inverse():
    rng = np.random.default_rng(0)
    for n in (64, 37, 16, 5):
        A = np.tril(0.3 * rng.standard_normal((n, n)), -1)
        T = blocked_unit_lower_inverse(A)
        np.testing.assert_allclose(T @ (np.eye(n) + A), np.eye(n), atol=1e-12)


CASES = [
    dict(B=2, T=150, Hqk=2, Hv=2, Dk=16, Dv=32, g_scale=0.1, init_std=0.3, beta_scale=2.0),
    dict(B=1, T=64, Hqk=2, Dk=16, dtype="f32"),
    dict(B=1, T=100, Hqk=1, Hv=3, Dk=32, Dv=16, g_scale=1.0, init_std=1.0),
    dict(B=1, Hqk=2, Hv=4, Dk=16, Dv=16, seqlens=[70, 0, 1, 64, 129], g_scale=0.05,
         init_std=0.02, beta_scale=2.0),
]


@pytest.mark.parametrize("case", range(len(CASES)))
@pytest.mark.parametrize("C", [16, 32, 64])
def test_chunked_equals_recurrence(case, C):
    x = make_case(dtype=CASES[case].get("dtype", "f32"),
                  **{kk: vv for kk, vv in CASES[case].items() if kk != "dtype"})
    f = x.f64()
    o_ref, s_ref = oracle.recurrent(f["q"], f["k"], f["v"], f["beta"], f["g"], f["init"],
                                    x.cu_seqlens, scale=0.5)
    o, s = chunked(f["q"], f["k"], f["v"], f["beta"], f["g"], f["init"], x.cu_seqlens,
                   scale=0.5, C=C)
    assert rel_l2(o, o_ref) < 1e-12
    assert rel_l2(s, s_ref) < 1e-12


def _bf16(x):
    return bf16_bits_to_f32(f32_to_bf16_bits(np.asarray(x, dtype=np.float32))).astype(np.float64)


def test_bf16_operand_rounding_error_budget():
    """Rounding every matrix-core operand to bf16 (as the GPU path does) keeps the
    relative L2 error well inside the 1e-2 bf16 tolerance on a (0, 2)-beta gated case
    (about 3e-3 here; rounding the fp64 output itself to bf16 alone costs 1.7e-3)."""
    x = make_case(B=1, T=512, Hqk=1, Hv=2, Dk=128, Dv=128, dtype="bf16", beta_scale=2.0,
                  g_scale=0.05, init_std=0.02, seed=4)
    f = x.f64()
    o_ref, s_ref = oracle.recurrent(f["q"], f["k"], f["v"], f["beta"], f["g"], f["init"])
    o, s = chunked(f["q"], f["k"], f["v"], f["beta"], f["g"], f["init"], quant=_bf16)
    assert rel_l2(o, o_ref) < 5e-3
    assert rel_l2(s, s_ref) < 5e-3


@pytest.mark.parametrize("C", [16, 64])
@pytest.mark.parametrize("gated", [False, True])
def test_chunked_backward_matches_oracle(C, gated):
    """The chunkwise reverse-pass algebra against the fp64 token-by-token reverse pass:
    packed sequences (an empty one, ragged chunks), GQA, beta in (0, 2), initial state."""
    from oracle.backward import backward
    from tests.chunk_model import chunked_backward
    x = make_case(B=1, Hqk=1, Hv=2, Dk=8, Dv=6, seqlens=[70, 0, 33, 5], g_scale=0.3 if gated else None,
                  init_std=0.5, beta_scale=2.0, seed=21)
    f = x.f64()
    rng = np.random.default_rng(22)
    do = rng.standard_normal((1, x.T, 2, 6))
    dfin = rng.standard_normal((x.num_seqs, 2, 8, 6))
    ref = backward(f["q"], f["k"], f["v"], f["beta"], f["g"], f["init"], do, dfin, x.cu_seqlens, 0.7)
    got = chunked_backward(f["q"], f["k"], f["v"], f["beta"], f["g"], f["init"], do, dfin,
                           x.cu_seqlens, 0.7, C=C)
    for name in ("dq", "dk", "dv", "dbeta", "dinit") + (("dg",) if gated else ()):
        np.testing.assert_allclose(got[name], ref[name], rtol=1e-9, atol=1e-9, err_msg=name)
