"""Planted mistakes in a copy of the oracle must each fail at least one pin.

Each mutant is a textual edit of oracle/oracle.c (a dropped term, a wrong sign,
a wrong index, a transposed layout, an off-by-one), compiled on the CPU into a
temporary library. The real oracle is never modified.
"""
import inspect
import os
import subprocess

import pytest

import oracle
import oracle_pins

SRC = os.path.join(os.path.dirname(oracle.__file__), "oracle.c")

MUTANTS = {
    "drop_scale": ("return scale * dot;", "return dot;"),
    "exp_sign": ("const double w = exp(work[j] - m);\n                const uint16_t",
                 "const double w = exp(m - work[j]);\n                const uint16_t"),
    "head_map_mod": ("const int g = h / G;", "const int g = h % n_kv_head;"),
    "layout_head_major": (
        "return (((size_t)b * (size_t)max_ctx + (size_t)p) * (size_t)n_kv_head +\n"
        "            (size_t)g) * (size_t)head_dim;",
        "return (((size_t)b * (size_t)n_kv_head + (size_t)g) * (size_t)max_ctx +\n"
        "            (size_t)p) * (size_t)head_dim;"),
    "live_off_by_one": ("long long n = (long long)position + 1;",
                        "long long n = (long long)position;"),
    "clamp_top_short": ("if (n > max_ctx) n = max_ctx;",
                        "if (n > max_ctx) n = max_ctx - 1;"),
    "chunk_floor": ("chunk = ((long long)nkv + n_splits - 1) / n_splits;",
                    "chunk = ((long long)nkv + n_splits) / n_splits;"),
    "combine_unweighted_S": ("S += w * r[1];", "S += r[1];"),
    "combine_weight_sign": ("exp(r[0] - gmx)", "exp(gmx - r[0])"),
    "f16_subnormal_scale": ("mag = ldexp((double)f, -24);",
                            "mag = ldexp((double)f, -25);"),
    "f16_bias": ("mag = ldexp(1024.0 + (double)f, e - 25);",
                 "mag = ldexp(1024.0 + (double)f, e - 24);"),
    "no_normalise": ("for (int d = 0; d < head_dim; ++d) o[d] /= denom;", ""),
    "partial_S_dropped": ("r[1] = S;", ""),
    "partial_no_max_shift": (
        "const double w = exp(work[j] - m);\n                    const uint16_t",
        "const double w = exp(work[j]);\n                    const uint16_t"),
    "score_first_dim_only": ("for (int d = 0; d < head_dim; ++d)\n        dot +=",
                             "for (int d = 0; d < 1; ++d)\n        dot +="),
    "f16_round_half_up": ("rint(a / quantum) * quantum", "floor(a / quantum + 0.5) * quantum"),
    "f16_truncate": ("rint(a / quantum) * quantum", "floor(a / quantum) * quantum"),
    "f16_subnormal_start": ("if (a == 0.0 || e < -14) e = -14;",
                            "if (a == 0.0 || e < -15) e = -15;"),
    "f16_nan_to_inf": ("if (isnan(v)) return (uint16_t)(sign | 0x7E00u);",
                       "if (isnan(v)) return (uint16_t)(sign | 0x7C00u);"),
    "append_row_offset": ("const long long p = (long long)positions[b] - (n_rows - 1) + t;",
                          "const long long p = (long long)positions[b] + t - n_rows;"),
    "append_drops_last_row": ("if (p < 0 || p >= max_ctx) continue;",
                              "if (p < 0 || p >= max_ctx - 1) continue;"),
    "append_k_from_v": ("k_cache[dst + i] = oracle_f32_to_f16(k_new[src + i]);",
                        "k_cache[dst + i] = oracle_f32_to_f16(v_new[src + i]);"),
    "rows_no_causal": ("long long p = (long long)positions[b] - (n_q - 1 - t);",
                       "long long p = (long long)positions[b];"),
    "rows_shift": ("long long p = (long long)positions[b] - (n_q - 1 - t);",
                   "long long p = (long long)positions[b] - (n_q - t);"),
    "rows_reversed": ("const size_t qi = ((size_t)b * n_q + t) * qrows;",
                      "const size_t qi = ((size_t)b * n_q + (n_q - 1 - t)) * qrows;"),
}

PINS = [f for n, f in inspect.getmembers(oracle_pins, inspect.isfunction)
        if n.startswith("pin_")]


@pytest.mark.parametrize("name", sorted(MUTANTS))
def test_mutant_is_caught(tmp_path, name):
    old, new = MUTANTS[name]
    with open(SRC) as f:
        text = f.read()
    assert old in text, f"mutation site for {name} not found"
    mutated = text.replace(old, new)
    src = tmp_path / "oracle.c"
    src.write_text(mutated)
    so = tmp_path / "liboracle_mutant.so"
    subprocess.run(["gcc", "-O2", "-std=c11", "-fPIC", "-shared", "-o", str(so),
                    str(src), "-lm"], check=True)
    lib = oracle.load(str(so))
    failed = []
    for pin in PINS:
        try:
            pin(lib)
        except AssertionError:
            failed.append(pin.__name__)
    assert failed, f"mutant {name} passed every pin"
