"""Mutation check of the FP8 oracle pins: each plausible mistake, planted into a
private copy of the oracle source on the CPU, must make at least one pin fail."""
import os
import subprocess

import pytest

import oracle
from tests import oracle_fp8_pins as P

HERE = os.path.dirname(oracle.__file__)
SRC = os.path.join(HERE, "attn_fp8_ref.c")
FWD_SRC = os.path.join(HERE, "attn_ref.c")

MUTATIONS = {
    "exponent_bias": ("ldexp(8.0 + m, e - 10)", "ldexp(8.0 + m, e - 11)"),
    "subnormal_scale": ("ldexp((double)m, -9)", "ldexp((double)m, -10)"),
    "nan_rule": ("if (e == 15 && m == 7) return NAN;", "if (e == 15) return NAN;"),
    "mantissa_hidden_bit": ("ldexp(8.0 + m, e - 10)", "ldexp(7.0 + m, e - 10)"),
    "drop_v_descale": ("orow[d] += p[j] * (s_v * e4m3_decode(vp[(size_t)j * D + d]));",
                       "orow[d] += p[j] * e4m3_decode(vp[(size_t)j * D + d]);"),
    "k_descale_twice": ("dot += qr[d] * (s_k * e4m3_decode(kp[(size_t)j * D + d]));",
                        "dot += qr[d] * (s_k * s_k * e4m3_decode(kp[(size_t)j * D + d]));"),
    "gqa_modulo": ("const int kvh = h / group;", "const int kvh = h % H_kv;"),
    "lse_without_max": ("lse[t] = m + log(l);", "lse[t] = log(l);"),
    "causal_off_by_one": ("const int nkeys = causal ? i + 1 : N;", "const int nkeys = causal ? i : N;"),
    "mag_signed": ("const double dev = w * fabs(", "const double dev = w * ("),
    "rms_not_squared": ("if (rrow) rrow[d] += dev * dev;", "if (rrow) rrow[d] += dev;"),
    "rms_no_root": ("rrow[d] = sqrt(rrow[d]);", "rrow[d] = rrow[d];"),
    "mag_floor_ignored": ("const double small = p[j] < w_floor ? p[j] : w_floor;",
                          "const double small = 0.0;"),
    "mag_unnormalised": ("const double w = (w_rel * p[j] > small ? w_rel * p[j] : small) / l;",
                         "const double w = (w_rel * p[j] > small ? w_rel * p[j] : small);"),
}


def _run_pins(fref, dec):
    failed = []
    for pin in P.ALL_PINS:
        try:
            pin(fref, dec)
        except (AssertionError, ValueError, FloatingPointError):
            failed.append(pin.__name__)
    return failed


@pytest.mark.parametrize("name", sorted(MUTATIONS))
def test_planted_mistake_is_caught(name, tmp_path):
    old, new = MUTATIONS[name]
    src = open(SRC).read()
    assert src.count(old) == 1, f"mutation anchor for {name} not found exactly once"
    path_c = tmp_path / f"mut_{name}.c"
    path_so = tmp_path / f"libmut_{name}.so"
    path_c.write_text(src.replace(old, new))
    subprocess.run(["gcc", "-O2", "-std=c11", "-fPIC", "-shared", "-pthread", "-o",
                    str(path_so), FWD_SRC, str(path_c), "-lm"], check=True)
    lib = oracle._bind(str(path_so))

    def fref(q8, k8, v8, dq, dk, dv, causal, scale, rows=None, mags=None):
        return oracle.call_fp8_lib(lib, q8, k8, v8, dq, dk, dv, causal, scale, rows, mags)

    def dec(codes):
        return oracle.call_e4m3_decode(lib, codes)

    assert _run_pins(fref, dec), f"no pin caught the planted mistake '{name}'"
