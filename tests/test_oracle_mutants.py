"""Plant a plausible mistake in a copy of the oracle (on the CPU) and check that
at least one pin catches it: the pins are strong enough to trust the oracle."""
import os
import subprocess
import sys

import pytest

import oracle as O

SRC = os.path.join(os.path.dirname(O.__file__), "oracle.c")
ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))

# (name, original text, mutated text, which occurrence)
MUTANTS = [
    ("pool_drops_last_token", "t < (i + 1) * B", "t < (i + 1) * B - 1", 0),
    ("pool_skips_first_token", "int t = i * B;", "int t = i * B + 1;", 0),
    ("pool_sum_not_mean", "xb[((int64_t)h * nb + i) * d + c] = sum * inv_b;",
     "xb[((int64_t)h * nb + i) * d + c] = sum;", 0),
    ("score_gqa_modulo", "int g = h / G;\n        for (int i = 0; i < nb; ++i) {",
     "int g = h % Hkv;\n        for (int i = 0; i < nb; ++i) {", 0),
    ("score_scale_1_over_d", "float sigma = (float)(1.0 / sqrt((double)d));",
     "float sigma = (float)(1.0 / (double)d);", 0),
    ("softmax_unnormalised", "prow[j] = prow[j] / sum;", "prow[j] = prow[j];", 0),
    ("score_transposed_kb", "const float *b = kb + ((int64_t)g * nb + j) * d;",
     "const float *b = kb + ((int64_t)g * nb + j);", 0),
    ("keep_count_floor", "return (int64_t)((num + ten_e - 1) / ten_e);",
     "return (int64_t)(num / ten_e);", 0),
    ("keep_count_binary_s", "if (strtod(b, NULL) != s)", "if (p < 17)", 0),
    ("select_ascending", "if (va > vb) return -1;", "if (va < vb) return -1;", 0),
    ("select_ties_highest_index", "return (a < b) ? -1 : (a > b);",
     "return (a > b) ? -1 : (a < b);", 0),
    ("select_keeps_one_less", "for (int64_t r = 0; r < K && r < n; ++r)",
     "for (int64_t r = 1; r < K && r < n; ++r)", 0),
    ("per_head_reads_head_0", "oracle_select(P + h * per, per, k_h, keep + h * per);",
     "oracle_select(P, per, k_h, keep + h * per);", 0),
    ("per_head_build_uses_global", "oracle_select_per_head(p_out, H, nb, k_h, keep);",
     "oracle_select(p_out, n, K, keep);", 0),
    ("per_head_budget_total", "oracle_select(P + h * per, per, k_h, keep + h * per);",
     "oracle_select(P + h * per, per, k_h * H, keep + h * per);", 0),
    ("csr_transposed", "if (keep[(int64_t)r * nb + j])", "if (keep[(int64_t)j * nb + r])", 0),
    ("plan_ascending", "if (la > lb) return -1;", "if (la < lb) return -1;", 0),
    ("plan_most_loaded_die", "load[x] < load[best]", "load[x] > load[best]", 0),
    ("plan_heads_ascending",
     "if (g_head_weight[a] > g_head_weight[b]) return -1;\n    if (g_head_weight[a] < g_head_weight[b]) return 1;",
     "if (g_head_weight[a] > g_head_weight[b]) return 1;\n    if (g_head_weight[a] < g_head_weight[b]) return -1;", 0),
    ("plan_empty_rows_reversed", "                    out[pos++] = h * nb + i;",
     "                    out[pos++] = h * nb + (nb - 1 - i);", 0),
    ("plan_empty_rows_dropped", "if (row_ptr[h * nb + i + 1] <= row_ptr[h * nb + i])",
     "if (row_ptr[h * nb + i + 1] < row_ptr[h * nb + i])", 0),
    ("plan_weight_kept_only", "weight[h] = (B / 32) * kept + 4 * rows;", "weight[h] = kept;", 0),
    ("plan_weight_no_row_cost", "weight[h] = (B / 32) * kept + 4 * rows;", "weight[h] = (B / 32) * kept;", 0),
    ("plan_weight_steps_ignore_block", "weight[h] = (B / 32) * kept + 4 * rows;", "weight[h] = 2 * kept + 4 * rows;", 0),
    ("attn_block_index_not_scaled", "toks[ntok++] = col_idx[e] * B + t;",
     "toks[ntok++] = col_idx[e] + t;", 0),
    ("attn_no_scale", "double scale = 1.0 / sqrt((double)d);", "double scale = 1.0;", 0),
    ("attn_unnormalised", "double p = z[a] / l;", "double p = z[a];", 0),
    ("attn_gqa_modulo", "int h = r / nb, i = r % nb, g = h / G;",
     "int h = r / nb, i = r % nb, g = h % Hkv;", 0),
    ("dense_gqa_modulo", "int h = r / nb, i = r % nb, g = h / G;",
     "int h = r / nb, i = r % nb, g = h % Hkv;", 1),
    ("attn_wrong_query_block", "for (int t = i * B; t < (i + 1) * B; ++t)\n            attend_token(q + ((int64_t)h * L + t) * d, kh, vh, d, toks, ntok",
     "for (int t = i * B; t < (i + 1) * B; ++t)\n            attend_token(q + ((int64_t)h * L + (t + B) % L) * d, kh, vh, d, toks, ntok", 0),
    ("mass_not_averaged", "arow[u / B] += z[u] / l / B;", "arow[u / B] += z[u] / l;", 0),
    ("mass_key_block_modulo", "arow[u / B] += z[u] / l / B;", "arow[u % nb] += z[u] / l / B;", 0),
    ("mass_gqa_modulo", "int h = r / nb, i = r % nb, g = h / G;\n        const float *kh = k + (int64_t)g * L * d;\n        double *arow",
     "int h = r / nb, i = r % nb, g = h % Hkv;\n        const float *kh = k + (int64_t)g * L * d;\n        double *arow", 0),
    ("recall_skips_last", "for (int32_t e = row_ptr[r]; e < row_ptr[r + 1]; ++e)",
     "for (int32_t e = row_ptr[r]; e + 1 < row_ptr[r + 1]; ++e)", 0),
    ("driver_period_from_zero", "since % refresh_every == 0", "step % refresh_every == 0", 0),
    ("bf16_truncates", "u = (u + 0x7FFFu + ((u >> 16) & 1u)) & 0xFFFF0000u;",
     "u = u & 0xFFFF0000u;", 0),
    ("bf16_ties_up", "u = (u + 0x7FFFu + ((u >> 16) & 1u)) & 0xFFFF0000u;",
     "u = (u + 0x8000u) & 0xFFFF0000u;", 0),
    ("col_pooled_not_rounded", "qb[x] = bf16_round(qb[x]);", "qb[x] = qb[x];", 0),
    ("col_mass_unnormalised", "ch[u] += z[u] / l / nb;", "ch[u] += z[u] / nb;", 0),
    ("col_mass_sum_not_mean", "ch[u] += z[u] / l / nb;", "ch[u] += z[u] / l;", 0),
    ("col_gqa_modulo", "int g = h / G;\n        const float *kh = k + (int64_t)g * L * d;\n        double *ch",
     "int g = h % Hkv;\n        const float *kh = k + (int64_t)g * L * d;\n        double *ch", 0),
    ("col_select_head_0", "oracle_select(c + (int64_t)h * L, L, k_c, keep);",
     "oracle_select(c, L, k_c, keep);", 0),
    ("col_attn_head_0_columns", "cols + (int64_t)h * k_c, (int)k_c, z,", "cols, (int)k_c, z,", 0),
    ("col_recall_not_averaged", "recall[r] = acc / B;", "recall[r] = acc;", 0),
    ("col_recall_head_0_columns", "const int32_t *ch = cols + (int64_t)h * k_c;",
     "const int32_t *ch = cols;", 0),
    ("col_recall_normalised_over_kept", "            for (int u = 0; u < L; ++u)\n                l += exp(z[u] - m);",
     "            for (int64_t a = 0; a < k_c; ++a)\n                l += exp(z[ch[a]] - m);", 0),
    ("col_attn_drops_last_column", "cols + (int64_t)h * k_c, (int)k_c, z,",
     "cols + (int64_t)h * k_c, (int)k_c - 1, z,", 0),
]


def _replace_nth(text, old, new, n):
    start = -1
    for _ in range(n + 1):
        start = text.index(old, start + 1)
    return text[:start] + new + text[start + len(old):]


@pytest.mark.parametrize("name,old,new,nth", MUTANTS, ids=[m[0] for m in MUTANTS])
def test_mutant_is_caught(name, old, new, nth, tmp_path):
    text = open(SRC).read()
    assert text.count(old) > nth, f"mutation site for {name} not found"
    src = tmp_path / "oracle_mut.c"
    src.write_text(_replace_nth(text, old, new, nth))
    so = str(tmp_path / "liboracle_mut.so")
    subprocess.run(["gcc", *O.oracle._CFLAGS, str(src), "-o", so, "-lm"], check=True)
    # Run the pins in a child process: a mutant may also crash (that counts as caught).
    script = (
        "import sys; sys.path[:0] = [%r, %r]\n"
        "import oracle as O, oracle_pins as pins\n"
        "lib = O.load(%r)\n"
        "failed = []\n"
        "for pin in pins.ALL_PINS:\n"
        "    try:\n"
        "        pin(lib)\n"
        "    except Exception as e:\n"
        "        failed.append(pin.__name__)\n"
        "print('caught by:', failed)\n"
        "sys.exit(1 if failed else 0)\n"
    ) % (ROOT, os.path.join(ROOT, "tests"), so)
    r = subprocess.run([sys.executable, "-c", script], capture_output=True, text=True, timeout=300)
    assert r.returncode != 0, f"mutant {name} passed every pin: {r.stdout} {r.stderr}"
