"""Mutation check of the block-sparse pins: each plausible mistake, planted into
a private copy of the oracle source on the CPU, must make at least one pin fail."""
import os
import subprocess

import pytest

import oracle
from tests import oracle_blocksparse_pins as P

HERE = os.path.dirname(oracle.__file__)
SRC = os.path.join(HERE, "attn_blocksparse_ref.c")
DEPS = [os.path.join(HERE, n) for n in ("attn_ref.c", "attn_varlen_ref.c")]

MUTATIONS = {
    "query_block_of_next_row": ("+ i / block;", "+ (i + 1 < N ? i + 1 : i) / block;"),
    "key_block_off_by_one": ("if (!allowed[j / block] || (causal && j > i)) continue;",
                             "if (!allowed[(j + 1 < N ? j + 1 : j) / block] || (causal && j > i)) continue;"),
    "causal_ignored": ("if (!allowed[j / block] || (causal && j > i)) continue;",
                       "if (!allowed[j / block]) continue;"),
    "mask_head_ignored": ("(int64_t)(mask_heads == 1 ? 0 : h) * n_blocks", "(int64_t)0 * n_blocks"),
    "last_entry_dropped": ("for (int32_t x = kb_ptr[list]; x < kb_ptr[list + 1]; ++x)",
                           "for (int32_t x = kb_ptr[list]; x < kb_ptr[list + 1] - 1; ++x)"),
    "gqa_modulo": ("const int kvh = h / group;", "const int kvh = h % H_kv;"),
    "lse_without_max": ("lse[t] = m + log(l);", "lse[t] = log(l);"),
    "empty_rows_nan": ("        if (!seen) {\n            lse[t] = -INFINITY;\n            continue;\n        }\n", ""),
    "drop_scale": ("e[j] = scale * dot;", "e[j] = dot;"),
    "neg_inf_scores_skipped": ("if (!sees[j]) continue;", "if (!sees[j] || e[j] == -INFINITY) continue;"),
}


def _run_pins(bref):
    failed = []
    for pin in P.ALL_PINS:
        try:
            pin(bref)
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
                    str(path_so), *DEPS, str(path_c), "-lm"], check=True)
    lib = oracle._bind(str(path_so))

    def bref(q, k, v, kb_ptr, kb_idx, block, causal, scale, rows=None):
        return oracle.call_blocksparse_lib(lib, q, k, v, kb_ptr, kb_idx, block, causal, scale, rows)

    assert _run_pins(bref), f"no pin caught the planted mistake '{name}'"
