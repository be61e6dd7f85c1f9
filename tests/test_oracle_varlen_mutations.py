"""Mutation check of the packed-batch / window pins: each plausible mistake,
planted into a private copy of the oracle source on the CPU, must make at
least one pin fail."""
import os
import subprocess

import pytest

import oracle
from tests import oracle_varlen_pins as P

HERE = os.path.dirname(oracle.__file__)
SRC = os.path.join(HERE, "attn_varlen_ref.c")
FWD_SRC = os.path.join(HERE, "attn_ref.c")

MUTATIONS = {
    "left_off_by_one": ("if (left >= 0 && i - left > lo) lo = i - left;",
                        "if (left >= 0 && i - left + 1 > lo) lo = i - left + 1;"),
    "right_off_by_one": ("if (right >= 0 && i + right < hi) hi = i + right;",
                         "if (right >= 0 && i + right - 1 < hi) hi = i + right - 1;"),
    "crosses_sequences": ("int64_t lo = s0, hi = s1 - 1;", "int64_t lo = 0, hi = total - 1;"),
    "causal_ignored": ("if (causal && i < hi) hi = i;", ""),
    "window_sides_swapped": ("if (left >= 0 && i - left > lo) lo = i - left;\n                if (right >= 0 && i + right < hi) hi = i + right;",
                             "if (right >= 0 && i - right > lo) lo = i - right;\n                if (left >= 0 && i + left < hi) hi = i + left;"),
    "gqa_modulo": ("const int kvh = h / group;", "const int kvh = h % H_kv;"),
    "drop_scale": ("e[j - lo] = scale * dot;", "e[j - lo] = dot;"),
    "lse_without_max": ("lse[(size_t)h * total + i] = m + log(l);",
                        "lse[(size_t)h * total + i] = log(l);"),
    "max_guarded_at_minus_inf": ("e[j - lo] = exp(e[j - lo] - m);",
                                 "e[j - lo] = exp(e[j - lo] - (m == -INFINITY ? 0.0 : m));"),
}


def _run_pins(vref):
    failed = []
    for pin in P.ALL_PINS:
        try:
            pin(vref)
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

    def vref(q, k, v, cu, causal, scale, left=-1, right=-1):
        return oracle.call_varlen_lib(lib, q, k, v, cu, causal, scale, left, right)

    assert _run_pins(vref), f"no pin caught the planted mistake '{name}'"
