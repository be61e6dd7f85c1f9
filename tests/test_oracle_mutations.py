"""Mutation check of the pins: each plausible mistake, planted into a private
copy of the oracle source on the CPU, must make at least one pin fail.

This shows that the pins constrain every part of the oracle (scale, mask,
head map, max subtraction, normalisation, LSE, operand roles, indexing)
rather than re-deriving it.
"""
import os
import subprocess

import pytest

import oracle
from tests import oracle_pins as P

SRC = os.path.join(os.path.dirname(oracle.__file__), "attn_ref.c")

MUTATIONS = {
    "drop_scale": ("s[j] = jb->scale * dot;", "s[j] = dot;"),
    # non-finite inputs
    "max_guarded_at_minus_inf": ("s[j] = exp(s[j] - m);", "s[j] = exp(s[j] - (m == -INFINITY ? 0.0 : m));"),
    "zero_weights_skipped": ("const double p = s[j];", "const double p = s[j];\n        if (p == 0.0) continue;"),
    "causal_off_by_one": ("jb->causal ? i + 1 : N", "jb->causal ? (i + 2 < N ? i + 2 : N) : N"),
    "causal_excludes_diagonal": ("jb->causal ? i + 1 : N", "jb->causal ? (i > 0 ? i : 1) : N"),
    "gqa_modulo_map": ("const int64_t kvh = h / group;", "const int64_t kvh = h % jb->Hkv;"),
    "no_max_subtraction": ("s[j] = exp(s[j] - m);", "s[j] = exp(s[j]);"),
    "lse_log2": ("*lse_out = m + log(l);", "*lse_out = m + log2(l);"),
    "lse_without_max": ("*lse_out = m + log(l);", "*lse_out = log(l);"),
    "missing_normalisation": ("for (int d = 0; d < D; ++d) o_row[d] /= l;", ""),
    "k_as_v": ("const uint16_t *vp = jb->v +", "const uint16_t *vp = jb->k +"),
    "q_head_uses_kv_head": ("((b * jb->Hq + h) * (int64_t)N + i) * D",
                            "((b * jb->Hq + kvh) * (int64_t)N + i) * D"),
    "sign_flip_exp": ("s[j] = exp(s[j] - m);", "s[j] = exp(m - s[j]);"),
    "dot_truncated": ("for (int d = 0; d < D; ++d) dot +=", "for (int d = 0; d + 1 < D; ++d) dot +="),
    "v_row_index_transposed": ("const uint16_t *vj = vp + j * D;", "const uint16_t *vj = vp + (nkeys - 1 - j) * D;"),
}


def _run_pins(ref):
    failed = []
    for pin in P.ALL_PINS:
        try:
            pin(ref)
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
                    str(path_so), str(path_c), "-lm"], check=True)
    lib = oracle._bind(str(path_so))

    def ref(q, k, v, causal, scale, rows=None):
        return oracle.call_lib(lib, q, k, v, causal, scale, rows, n_threads=2)

    failed = _run_pins(ref)
    assert failed, f"no pin caught the planted mistake '{name}'"
