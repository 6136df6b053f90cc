"""The oracle's pins must catch plausible mistakes. Each case below plants one
mistake in a copy of the oracle's C source (on the CPU, in a temporary
directory), builds it, and runs the matching pin suite (forward or backward)
against that build: at least one pin must fail. The in-tree oracle is never
modified."""
import os
import subprocess
import sys

import pytest

import oracle

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))

# (name, [(text in the source, planted replacement), ...])
MUTANTS = [
    ("no_max_subtraction", [("exp(scratch[j] - best)", "exp(scratch[j])"),
                            ("exp(row[j] - best)", "exp(row[j])"),
                            ("best + log(total)", "log(total)")]),
    ("causal_excludes_diagonal", [("causal ? (i + 1) : T", "causal ? i : T")]),
    ("causal_one_too_many", [("causal ? (i + 1) : T",
                              "causal ? (i + 2 < T ? i + 2 : T) : T")]),
    ("key_operand_transposed", [("(double)k[j * D + e]", "(double)k[e * T + j]")]),
    ("scale_dropped", [("const double s = scale * dot;", "const double s = dot;"),
                       ("row[j] = scale * dot;", "row[j] = dot;")]),
    ("scale_applied_twice", [("const double s = scale * dot;",
                              "const double s = scale * scale * dot;")]),
    ("lse_base_two", [("best + log(total)", "best + log2(total)")]),
    ("no_normalisation", [("o_row[e] /= total;", "o_row[e] /= 1.0;"),
                          ("row[j] /= total;", "row[j] /= 1.0;")]),
    ("value_row_fixed", [("v + j * D;", "v;")]),
    ("value_weight_sign", [("o_row[e] += w * (double)vj[e];",
                            "o_row[e] -= w * (double)vj[e];")]),
    ("sum_drops_first_key", [("for (int64_t j = 0; j < visible; ++j) {\n"
                              "        const double w = exp(",
                              "for (int64_t j = 0; j < visible; ++j) {\n"
                              "        if (j == 0) { scratch[j] = 0; continue; }\n"
                              "        const double w = exp(")]),
]


# mistakes in the backward pass, checked against the backward's pins
BACKWARD_MUTANTS = [
    ("bwd_no_delta", [("*dS = *P * (dpv - delta[i]);", "*dS = *P * dpv;")]),
    ("bwd_ds_sign", [("*dS = *P * (dpv - delta[i]);", "*dS = *P * (delta[i] - dpv);")]),
    ("bwd_dq_scale_dropped", [("for (int64_t e = 0; e < D; ++e) g[e] *= scale;",
                               "for (int64_t e = 0; e < D; ++e) g[e] *= 1.0;")]),
    ("bwd_dk_scale_dropped", [("for (int64_t e = 0; e < D; ++e) gk[e] *= scale;",
                               "for (int64_t e = 0; e < D; ++e) gk[e] *= 1.0;")]),
    ("bwd_dv_from_ds", [("gv[e] += P * (double)ds[i * D + e];",
                         "gv[e] += dS * (double)ds[i * D + e];")]),
    ("bwd_dk_key_operand", [("gk[e] += dS * (double)qs[i * D + e];",
                             "gk[e] += dS * (double)ks[i * D + e];")]),
    ("bwd_dk_sees_masked_rows", [("for (int64_t i = causal ? j : 0; i < T; ++i) {",
                                  "for (int64_t i = 0; i < T; ++i) {")]),
    ("bwd_p_without_lse", [("*P = exp(scale * dot - lse[i]);", "*P = exp(scale * dot);")]),
    ("bwd_dp_key_operand", [("dpv += (double)dout[i * D + e] * (double)v[j * D + e];",
                             "dpv += (double)dout[i * D + e] * (double)k[j * D + e];")]),
    ("bwd_delta_from_values", [("d += (double)ds[i * D + e] * o_row[e];",
                                "d += (double)ds[i * D + e] * (double)vs[i * D + e];")]),
]

# mistakes in the decode alignment, checked against the decode pins
DECODE_MUTANTS = [
    ("kv_top_left", [("causal, scale, Tk - Tq + i, scratch", "causal, scale, i, scratch")]),
    ("kv_one_early", [("causal, scale, Tk - Tq + i, scratch",
                       "causal, scale, Tk - Tq + i - (i > 0), scratch")]),
    ("kv_one_late", [("causal, scale, Tk - Tq + i, scratch",
                      "causal, scale, (Tk - Tq + i + 1 < Tk ? Tk - Tq + i + 1 : Tk - 1), scratch")]),
    ("kv_wrong_slice", [("k + slice * Tk * D, v + slice * Tk * D",
                         "k + slice * Tq * D, v + slice * Tq * D")]),
]

# mistakes in the gated linear recurrence
RECURRENCE_MUTANTS = [
    ("rec_gate_on_rows", [("S[i * D + j] = (double)gate[row + j] * S[i * D + j] +",
                           "S[i * D + j] = (double)gate[row + i] * S[i * D + j] +")]),
    ("rec_gate_after_add", [("S[i * D + j] = (double)gate[row + j] * S[i * D + j] +\n"
                             "                                   (double)k[row + i] * (double)v[row + j];",
                             "S[i * D + j] = (double)gate[row + j] * (S[i * D + j] +\n"
                             "                                   (double)k[row + i] * (double)v[row + j]);")]),
    ("rec_outer_transposed", [("(double)k[row + i] * (double)v[row + j];",
                               "(double)k[row + j] * (double)v[row + i];")]),
    ("rec_readout_wrong_index", [("acc += (double)q[row + i] * S[i * D + j];",
                                  "acc += (double)q[row + i] * S[j * D + i];")]),
    ("rec_readout_with_key", [("acc += (double)q[row + i] * S[i * D + j];",
                               "acc += (double)k[row + i] * S[i * D + j];")]),
    ("rec_state_not_reset", [("double* S = (double*)calloc((size_t)(D * D), sizeof(double));",
                              "static double Sbuf[4096]; double* S = D * D <= 4096 ? Sbuf : "
                              "(double*)calloc((size_t)(D * D), sizeof(double));"),
                             ("        free(S);\n    }\n    (void)nthreads;\n    return failed",
                              "        if (S != Sbuf) free(S);\n    }\n    (void)nthreads;\n"
                              "    return failed")]),
]

CASES = [(n, e, "test_oracle_pins.py") for n, e in MUTANTS] + \
    [(n, e, "test_oracle_bwd_pins.py") for n, e in BACKWARD_MUTANTS] + \
    [(n, e, "test_oracle_kv_pins.py") for n, e in DECODE_MUTANTS] + \
    [(n, e, "test_oracle_recurrence_pins.py") for n, e in RECURRENCE_MUTANTS]


@pytest.mark.parametrize("name,edits,pins", CASES, ids=[c[0] for c in CASES])
def test_pins_catch_mutant(name, edits, pins, tmp_path):
    src = open(oracle.SOURCE).read()
    for old, new in edits:
        assert old in src, f"mutation site {old!r} not found"
        src = src.replace(old, new)
    csrc = tmp_path / "mutant.c"
    csrc.write_text(src)
    lib = tmp_path / "libmutant.so"
    subprocess.run(["gcc", *oracle.CFLAGS, "-o", str(lib), str(csrc), "-lm"],
                   check=True)
    env = dict(os.environ, ATTN_ORACLE_LIBRARY=str(lib))
    r = subprocess.run([sys.executable, "-m", "pytest", "-x", "-q",
                        "-p", "no:cacheprovider",
                        os.path.join(ROOT, "tests", pins)],
                       cwd=ROOT, env=env, capture_output=True, text=True,
                       timeout=600)
    assert r.returncode != 0, f"mutant {name} passed every pin:\n{r.stdout[-2000:]}"
    assert "failed" in r.stdout, r.stdout[-2000:] + r.stderr[-2000:]
