"""Mutation check of the backward pins: each plausible mistake, planted into a
private copy of the backward oracle source on the CPU, must make at least one
pin fail (delta term, signs, scales, operand roles, masks, group sums, the
softmax normaliser, the error-scale sums)."""
import os
import subprocess

import pytest

import oracle
from tests import oracle_bwd_pins as P

HERE = os.path.dirname(oracle.__file__)
SRC = os.path.join(HERE, "attn_bwd_ref.c")
FWD_SRC = os.path.join(HERE, "attn_ref.c")

MUTATIONS = {
    "row_drops_delta": ("const double ds = p[j] * (dp[j] - delta);",
                        "const double ds = p[j] * dp[j];"),
    "key_drops_delta": ("const double ds = p * (dp - c->delta[r]);",
                        "const double ds = p * dp;"),
    "delta_sign": ("delta += p[j] * dot;", "delta -= p[j] * dot;"),
    "dq_missing_scale": ("dq_row[d] *= c->scale;", ""),
    "dk_missing_scale": ("dk[d] *= c->scale;", ""),
    "dk_uses_k": ("dk[d] += ds * qrow[d];", "dk[d] += ds * bwd_widen(kj[d]);"),
    "dv_uses_v": ("dv[d] += p * dorow[d];", "dv[d] += p * bwd_widen(vj[d]);"),
    "dv_uses_ds": ("dv[d] += p * dorow[d];", "dv[d] += ds * dorow[d];"),
    "gqa_first_head_only": ("h < (kvh + 1) * group; ++h) {\n        const int64_t first_row",
                            "h < kvh * group + 1; ++h) {\n        const int64_t first_row"),
    "gqa_modulo_map": ("const int64_t kvh = h / (c->Hq / c->Hkv);",
                       "const int64_t kvh = h % c->Hkv;"),
    "key_mask_off": ("const int64_t first_row = c->causal ? j : 0;",
                     "const int64_t first_row = 0;"),
    "key_mask_off_by_one": ("const int64_t first_row = c->causal ? j : 0;",
                            "const int64_t first_row = c->causal ? j + 1 : 0;"),
    "p_without_lse": ("exp(c->scale * s - c->lse[r])", "exp(c->scale * s)"),
    "p_without_scale": ("exp(c->scale * s - c->lse[r])", "exp(s - c->lse[r])"),
    "lse_log2": ("c->lse[slot] = m + log(l);", "c->lse[slot] = m + log2(l);"),
    "dp_uses_k": ("const double vjd = bwd_widen(vp[j * D + d]);",
                  "const double vjd = bwd_widen(kp[j * D + d]);"),
    "dq_uses_v": ("const double kjd = bwd_widen(kp[j * D + d]);",
                  "const double kjd = bwd_widen(vp[j * D + d]);"),
    "no_normalisation": ("for (int64_t j = 0; j < nkeys; ++j) p[j] /= l;", ""),
    "row_mask_off_by_one": ("const int64_t nkeys = c->causal ? i + 1 : N;",
                            "const int64_t nkeys = c->causal ? (i > 0 ? i : 1) : N;"),
    "dq_key_index_reversed": ("const double kjd = bwd_widen(kp[j * D + d]);",
                              "const double kjd = bwd_widen(kp[(nkeys - 1 - j) * D + d]);"),
    "mag_dv_signed": ("if (mdv) mdv[d] += p * fabs(dorow[d]);",
                      "if (mdv) mdv[d] += p * dorow[d];"),
    "keys_mode_skips_group": ("for (int64_t h = kvh * group; h < (kvh + 1) * group; ++h)\n            for (int64_t i = first[u]; i < N; ++i) rows[n_rows++]",
                              "for (int64_t h = kvh * group; h < kvh * group + 1; ++h)\n            for (int64_t i = first[u]; i < N; ++i) rows[n_rows++]"),
    "keys_mode_first_row_past_key": ("const int64_t f = causal ? j : 0;",
                                     "const int64_t f = causal ? j + 1 : 0;"),
    "keys_mode_skips_rows_noncausal": ("const int64_t f = causal ? j : 0;",
                                       "const int64_t f = j;"),
    "mag_dq_drops_k_abs": ("if (mdq_row) mdq_row[d] += w * fabs(kjd);",
                           "if (mdq_row) mdq_row[d] += w * kjd;"),
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
                    str(path_so), FWD_SRC, str(path_c), "-lm"], check=True)
    lib = oracle._bind(str(path_so))

    def bref(q, k, v, do, causal, scale, rows=None, mags=False, keys=None):
        return oracle.call_bwd_lib(lib, q, k, v, do, causal, scale, rows, mags, n_threads=2,
                                   keys=keys)

    failed = _run_pins(bref)
    assert failed, f"no pin caught the planted mistake '{name}'"
