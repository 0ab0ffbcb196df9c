"""The oracle's pins catch plausible mistakes.

Each case plants one mistake in a copy of oracle.c (a dropped term, a wrong
sign or index, a swapped operand, a wrong rounding), builds it with gcc on the
CPU into a temporary library, and runs the pin suite against it in a child
process: the suite must fail for every mutant.
"""
import os
import subprocess
import sys

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
SRC = os.path.join(ROOT, "oracle", "oracle.c")

MUTANTS = {
    "dropped_scale": ("return scale * s;", "return s;"),
    "gqa_index_modulo": ("g = h / G, D = kv->D;", "g = h % kv->Hkv, D = kv->D;"),
    "page_slot_swapped": ("slot = jj % kv->page_size;", "slot = (jj + 1) % kv->page_size;"),
    "merge_alpha_sign": ("0.0 : exp(mi - m);", "0.0 : exp(m - mi);"),
    "lse_drops_max": ("lse[bh] = m + log(dsum);\n        }\n        free(sbuf);",
                      "lse[bh] = log(dsum);\n        }\n        free(sbuf);"),
    "rope_sign": ("x[i] = a * c - b * s;", "x[i] = a * c + b * s;"),
    "rope_frequency": ("pow(base, -2.0 * (double)i", "pow(base, -1.0 * (double)i"),
    "rope_pairing": ("double a = x[i], b = x[i + half];", "double a = x[i], b = x[i ^ 1];"),
    "f16_bias": ("ldexp((double)(m + 1024), e - 25)", "ldexp((double)(m + 1024), e - 24)"),
    "f16_truncates": ("double v = rint(a / ulp) * ulp; /* rint", "double v = floor(a / ulp) * ulp; /* rint"),
    "v_reads_k": ("p * elem(kv, kv->v, kv->v_descale, b, g, off + d);", "p * elem(kv, kv->k, kv->v_descale, b, g, off + d);"),
    "f8_bias_8": ("ldexp((double)(m + 8), e - 10)", "ldexp((double)(m + 8), e - 11)"),
    "f8_subnormal_scale": ("v = ldexp((double)m, -9);", "v = ldexp((double)m, -10);"),
    "f8_descale_dropped": ("((const uint8_t *)base)[off]) * f;", "((const uint8_t *)base)[off]);"),
    "f8_v_uses_k_descale": ("p * elem(kv, kv->v, kv->v_descale, b, g, off + d);", "p * elem(kv, kv->v, kv->k_descale, b, g, off + d);"),
    "f8_descale_index_swapped": ("descale[(int64_t)b * kv->Hkv + g]", "descale[(int64_t)g * kv->B + b]"),
    "last_token_dropped": ("for (int j = lo; j < hi; ++j) {\n        sbuf",
                           "for (int j = lo; j < hi - 1; ++j) {\n        sbuf"),
    "prefix_pages_ignored": ("} else if (kv->prefix_pages && j < kv->prefix_len) {",
                             "} else if (kv->prefix_pages && j < 0) {"),
    "append_v_not_written": ("for (int d = 0; d < D; ++d) vc[off + d] = vn[d];", ""),
    "f8_encode_ties_odd": ("(err == best_err && (c & 1) == 0)", "(err == best_err && (c & 1) == 1)"),
    "f8_encode_rounds_down": ("double err = fabs(oracle_f8_to_f64((uint8_t)c) - a);",
                              "double err = oracle_f8_to_f64((uint8_t)c) > a ? INFINITY : a - oracle_f8_to_f64((uint8_t)c);"),
    "f8_encode_drops_sign": ("return (uint8_t)(signbit(x) ? (best | 0x80) : best);", "return (uint8_t)best;"),
    "f8_encode_nan_saturates": ("if (isnan(x)) return 0x7f;", "if (isnan(x)) return 0x7e;"),
    "f8_append_multiplies_descale": ("kc[off + d] = oracle_f32_to_f8(x / kd);", "kc[off + d] = oracle_f32_to_f8(x * kd);"),
    "f8_append_v_uses_k_descale": ("vc[off + d] = oracle_f32_to_f8(y / vd);", "vc[off + d] = oracle_f32_to_f8(y / kd);"),
    "f8_append_k_unrotated": ("if (rotary_dim > 0) oracle_rope_neox(tmp, D, rotary_dim, pos, base);\n            if (f8) {",
                              "if (rotary_dim > 0 && !f8) oracle_rope_neox(tmp, D, rotary_dim, pos, base);\n            if (f8) {"),
    "batch_idx_ignored": ("outer = kv->batch_idx ? kv->batch_idx[b] : b;", "outer = b;"),
    "leftpad_ignored": ("int lo = first_row(kv, b);\n            double m, dsum;",
                        "int lo = 0;\n            double m, dsum;"),
    "multi_leftpad_ignored": ("int lo = first_row(kv, b);\n            int hi", "int lo = 0;\n            int hi"),
    "partials_ignore_leftpad": ("if (lo < first_row(kv, b)) lo = first_row(kv, b);", ""),
    "rope_at_row_not_position": ("int pos = c - first_row(kv, b);", "int pos = c;"),
    "causal_excludes_own_row": ("int hi = lens[b] - q_len + i + 1;", "int hi = lens[b] - q_len + i;"),
    "tokens_reversed": ("int hi = lens[b] - q_len + i + 1;", "int hi = lens[b] - i;"),
    "multi_lse_token_major": ("double *l = lse + ((int64_t)b * Hq + h) * q_len + i;",
                              "double *l = lse + ((int64_t)b * q_len + i) * Hq + h;"),
}


@pytest.mark.parametrize("name", sorted(MUTANTS))
def test_pins_reject_planted_mistake(name, tmp_path):
    old, new = MUTANTS[name]
    src = open(SRC).read()
    assert src.count(old) == 1, f"mutation site for {name} not unique"
    mut = tmp_path / "oracle_mut.c"
    mut.write_text(src.replace(old, new))
    lib = tmp_path / "liboracle_mut.so"
    subprocess.run(["gcc", "-O1", "-std=c11", "-fPIC", "-shared", "-fopenmp", str(mut), "-o",
                    str(lib), "-lm"], check=True)
    env = dict(os.environ, ORACLE_LIB_OVERRIDE=str(lib))
    r = subprocess.run([sys.executable, "-m", "pytest", "-x", "-q", "-p", "no:cacheprovider",
                        os.path.join(ROOT, "tests", "test_oracle.py")],
                       cwd=ROOT, env=env, capture_output=True, text=True, timeout=600)
    assert r.returncode != 0, f"pins did not catch mutant {name}:\n{r.stdout[-2000:]}"
