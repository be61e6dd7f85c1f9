"""Mutation check of the decode and merge pins: each plausible mistake, planted
into a private copy of the oracle source on the CPU, must make at least one pin
fail."""
import os
import subprocess

import pytest

import oracle
from tests import oracle_decode_pins as P

HERE = os.path.dirname(oracle.__file__)
SRC = os.path.join(HERE, "attn_decode_ref.c")
FWD_SRC = os.path.join(HERE, "attn_ref.c")

MUTATIONS = {
    "causal_off_by_one": ("const int nkeys = causal ? L - M + i + 1 : L;",
                          "const int nkeys = causal ? L - M + i : L;"),
    "causal_top_left": ("const int nkeys = causal ? L - M + i + 1 : L;",
                        "const int nkeys = causal ? i + 1 : L;"),
    "drop_scale": ("s[j] = scale * dot;", "s[j] = dot;"),
    "gqa_modulo": ("const int kvh = h / group;", "const int kvh = h % H_kv;"),
    "no_normalisation": ("for (int d = 0; d < D; ++d) orow[d] /= l;", ""),
    "lse_without_max": ("lse[r] = m + log(l);", "lse[r] = log(l);"),
    "merge_no_max_shift": ("for (int p = 0; p < n_parts; ++p) total += exp(lp[p] - m);\n        const double L = m + log(total);",
                           "for (int p = 0; p < n_parts; ++p) total += exp(lp[p]);\n        const double L = log(total);"),
    "merge_unnormalised_weight": ("const double w = exp(lp[p] - L);", "const double w = exp(lp[p] - m);"),
    "merge_lse_log2": ("const double L = m + log(total);", "const double L = m + log2(total);"),
    "merge_first_part_only": ("for (int p = 0; p < n_parts; ++p) {\n            const double w",
                              "for (int p = 0; p < 1; ++p) {\n            const double w"),
    "merge_max_ignores_last": ("for (int p = 0; p < n_parts; ++p) {\n            if (isnan(lp[p])) nan_part = 1;",
                               "for (int p = 0; p + 1 < n_parts; ++p) {\n            if (isnan(lp[p])) nan_part = 1;"),
    "merge_drops_nan_part": ("if (isnan(lp[p])) nan_part = 1;", "if (0) nan_part = 1;"),
}


def _run_pins(dref, mref):
    failed = []
    for pin in P.ALL_PINS:
        try:
            pin(dref, mref)
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

    def dref(q, k, v, causal, scale):
        return oracle.call_decode_lib(lib, q, k, v, causal, scale)

    def mref(op, lp):
        return oracle.call_merge_lib(lib, op, lp)

    failed = _run_pins(dref, mref)
    assert failed, f"no pin caught the planted mistake '{name}'"
