"""Plant plausible mistakes in copies of the oracle's C source and require that the pins
catch every one (a mistake the pins cannot see would leave the oracle unpinned).

Each mutant is compiled from a modified copy of oracle/dn_oracle.c into a temporary
folder; the real oracle is never touched.
"""
import functools
import os

import pytest

import oracle
from tests.oracle_pins import ALL_PINS

READ = """            /* o_t = scale * S_t q_t */
            double *ot = o + (t * Hv + h) * Dv;
            for (int64_t j = 0; j < Dv; ++j) {
                double s = 0.0;
                for (int64_t i = 0; i < Dk; ++i)
                    s += S[j * Dk + i] * qt[i];
                ot[j] = scale * s;
            }
"""
DECAY = """            /* decay first: S <- exp(g_t) S */
            if (g && gdim == 1) {
                const double a = exp(g[t * Hv + h]);
                for (int64_t e = 0; e < Dv * Dk; ++e)
                    S[e] *= a;
            }
            /* channel gates: S <- S diag(exp(g_t)), key channel i keeps exp(g_t[i]) */
            if (g && gdim != 1) {
                for (int64_t i = 0; i < Dk; ++i) {
                    const double a = exp(g[(t * Hv + h) * Dk + i]);
                    for (int64_t j = 0; j < Dv; ++j)
                        S[j * Dk + i] *= a;
                }
            }
"""
PRED = "            /* prediction error S k_t - v_t */\n"


def _move(src, block, before):
    assert src.count(block) == 1 and src.count(before) == 1
    src = src.replace(block, "")
    return src.replace(before, block + before)


def _sub(old, new):
    def f(src):
        assert src.count(old) == 1, old
        return src.replace(old, new)
    return f


MUTANTS = {
    "update_sign": _sub("S[j * Dk + i] -= bt * pred[j] * kt[i];", "S[j * Dk + i] += bt * pred[j] * kt[i];"),
    "error_sign": _sub("pred[j] = s - vt[j];", "pred[j] = s + vt[j];"),
    "beta_dropped": _sub("-= bt * pred[j] * kt[i];", "-= pred[j] * kt[i];"),
    "beta_squared": _sub("-= bt * pred[j] * kt[i];", "-= bt * bt * pred[j] * kt[i];"),
    "retrieve_with_query": _sub("s += S[j * Dk + i] * kt[i];", "s += S[j * Dk + i] * qt[i];"),
    "read_with_key": _sub("s += S[j * Dk + i] * qt[i];", "s += S[j * Dk + i] * kt[i];"),
    "scale_dropped": _sub("ot[j] = scale * s;", "ot[j] = s;"),
    "gate_linearised": _sub("const double a = exp(g[t * Hv + h]);", "const double a = 1.0 + g[t * Hv + h];"),
    "gate_sign": _sub("const double a = exp(g[t * Hv + h]);", "const double a = exp(-g[t * Hv + h]);"),
    "gate_previous_token": _sub("const double a = exp(g[t * Hv + h]);",
                                "const double a = exp(g[(t > cu[n] ? t - 1 : t) * Hv + h]);"),
    "init_not_transposed": _sub("S[j * Dk + i] = m0[i * Dv + j];", "S[j * Dk + i] = m0[j * Dk + i];"),
    "final_not_transposed": _sub("m1[i * Dv + j] = S[j * Dk + i];", "m1[j * Dk + i] = S[j * Dk + i];"),
    "qk_head_modulo": _sub("hq = h / group;", "hq = h % Hqk;"),
    "beta_of_qk_head": _sub("const double bt = beta[t * Hv + h];", "const double bt = beta[t * Hv + hq];"),
    "outer_uses_query": _sub("-= bt * pred[j] * kt[i];", "-= bt * pred[j] * qt[i];"),
    "read_before_write": lambda s: _move(s, READ, PRED),
    "decay_after_write": lambda s: _move(s, DECAY, "            /* o_t = scale * S_t q_t */\n"),
    "norm_eps_outside_sqrt": _sub("ik = 1.0 / sqrt(sk + eps)", "ik = 1.0 / (sqrt(sk) + eps)"),
    "norm_by_squared_norm": _sub("ik = 1.0 / sqrt(sk + eps)", "ik = 1.0 / (sk + eps)"),
    "norm_keys_only": _sub("iq = 1.0 / sqrt(sq + eps)", "iq = 1.0"),
    "norm_key_by_query": _sub("ik = 1.0 / sqrt(sk + eps)", "ik = 1.0 / sqrt(sq + eps)"),
    "norm_skipped": _sub("if (qk_l2norm) {", "if (0) {"),
    "channel_gate_reversed": _sub("const double a = exp(g[(t * Hv + h) * Dk + i]);",
                                  "const double a = exp(g[(t * Hv + h) * Dk + (Dk - 1 - i)]);"),
    "channel_gate_first_channel": _sub("const double a = exp(g[(t * Hv + h) * Dk + i]);",
                                       "const double a = exp(g[(t * Hv + h) * Dk]);"),
    "channel_gate_of_qk_head": _sub("const double a = exp(g[(t * Hv + h) * Dk + i]);",
                                    "const double a = exp(g[(t * Hv + hq) * Dk + i]);"),
    "channel_gate_sign": _sub("const double a = exp(g[(t * Hv + h) * Dk + i]);",
                              "const double a = exp(-g[(t * Hv + h) * Dk + i]);"),
    "skips_first_token": _sub("for (int64_t t = cu[n]; t < cu[n + 1]; ++t) {",
                              "for (int64_t t = cu[n] + 1; t < cu[n + 1]; ++t) {"),
}


@pytest.fixture(scope="module")
def source():
    with open(oracle.SRC) as f:
        return f.read()


@pytest.mark.parametrize("name", sorted(MUTANTS))
def test_mutant_is_caught(name, source, tmp_path):
    src = MUTANTS[name](source)
    assert src != source
    cpath = os.path.join(str(tmp_path), f"mut_{name}.c")
    with open(cpath, "w") as f:
        f.write(src)
    lib = oracle.compile_source(cpath, os.path.join(str(tmp_path), f"libmut_{name}.so"),
                                 werror=False)
    run = functools.partial(oracle.recurrent, lib_path=lib)
    caught = []
    for pin in ALL_PINS:
        try:
            pin(run)
        except (AssertionError, ValueError, FloatingPointError):
            caught.append(pin.__name__)
    assert caught, f"no pin catches the planted mistake {name!r}"
