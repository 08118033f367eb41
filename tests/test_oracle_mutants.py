"""Each plausible mistake planted in a copy of the oracle (on the CPU) is
caught by at least one pin. The planted copies live in a temporary directory;
the real oracle source is never touched."""

import pytest

import oracle
import oracle_pins as pins

MUTANTS = {
    "drop_last_k_term": ("k < K; ++k) {\n        double p", "k < K - 1; ++k) {\n        double p"),
    "wrong_sign": ("acc = acc + (float)p;\n        sabs += fabs(p);\n        ref += p;",
                   "acc = acc - (float)p;\n        sabs += fabs(p);\n        ref += p;"),
    "uv_wrong_sign": ("acc = acc + (float)p;\n          sabs += fabs(p);\n        }",
                      "acc = acc - (float)p;\n          sabs += fabs(p);\n        }"),
    "scale_index_by_k": ("+ n / ORACLE_MX_BLOCK];", "+ k / ORACLE_MX_BLOCK];"),
    "q_nope_as_HMK": ("j->q_nope + ((size_t)m * H + h) * K", "j->q_nope + ((size_t)h * j->M + m) * K"),
    "weight_as_HNK": ("size_t idx = ((size_t)h * j->K + k) * j->N + n;",
                      "size_t idx = ((size_t)h * j->N + n) * j->K + k;"),
    "q_pe_reversed": ("((uint16_t*)j->out)[orow + N + r] = pe[r];",
                      "((uint16_t*)j->out)[orow + N + r] = pe[R - 1 - r];"),
    "bf16_ties_away": ("return (lo & 1u) ? hi : lo;", "return hi;"),
    "e4m3_ties_odd": ("(d == bestd && (c & 1) == 0)", "(d == bestd && (c & 1) == 1)"),
    "e4m3_bias_off_by_one": ("ldexp((double)(8 + m), e - 10)", "ldexp((double)(8 + m), e - 11)"),
    "e8m0_bias_off_by_one": ("ldexp(1.0, (int)b - 127)", "ldexp(1.0, (int)b - 128)"),
    "multiply_by_q_scale": ("f32_to_e4m3_satfinite(v / q_scale)", "f32_to_e4m3_satfinite(v * q_scale)"),
    "e4m3_without_bf16_step": ("to_e4m3_out(bf16_to_f32(y), j->q_scale)", "to_e4m3_out(acc, j->q_scale)"),
    "q_pe_unscaled": ("to_e4m3_out(bf16_to_f32(pe[r]), j->q_scale)", "to_e4m3_out(bf16_to_f32(pe[r]), 1.0f)"),
    "uv_scale_indexed_by_v": ("* (C / ORACLE_MX_BLOCK) + c / ORACLE_MX_BLOCK];",
                              "* (C / ORACLE_MX_BLOCK) + v % (C / ORACLE_MX_BLOCK)];"),
    "uv_weight_as_HCV": ("size_t idx = ((size_t)h * V + v) * C + c;", "size_t idx = ((size_t)h * C + c) * V + v;"),
    "uv_drop_last_c": ("for (int c = 0; c < C; ++c) {\n          double p", "for (int c = 0; c < C - 1; ++c) {\n          double p"),
    "projection_offset_by_one": ("((uint16_t*)j->out)[orow + n] = y;", "((uint16_t*)j->out)[orow + (n + 1) % N] = y;"),
    "attn_scale_missing": ("s[t] = j->softmax_scale * acc;", "s[t] = acc;"),
    "attn_value_from_rope": ("o[d] += e * (double)bf16_to_f32(row[d]);",
                             "o[d] += e * (double)bf16_to_f32(row[d + (j->D - j->DV)]);"),
    "attn_drop_last_token": ("for (int t = a; t < b; ++t) {\n    double e", "for (int t = a; t < b - 1; ++t) {\n    double e"),
    "attn_row_off_by_one": ("(size_t)(t % j->P)) * j->D;", "(size_t)((t + 1) % j->P)) * j->D;"),
    "attn_split_align_32": ("#define ORACLE_SPLIT_ALIGN 64", "#define ORACLE_SPLIT_ALIGN 32"),
    "attn_merge_weight_inverted": ("double w = exp(plse[sp] - Lp);", "double w = exp(Lp - plse[sp]);"),
    "attn_bf16_partial_skipped": ("po[d] = (double)bf16_to_f32(f64_to_bf16_rne(po[d]));", "po[d] = (double)(float)po[d];"),
    "attn_lse_kept_double": ("if (j->partial_dtype != ORACLE_PARTIAL_EXACT) plse[sp] = (double)(float)plse[sp];", "(void)0;"),
    "attn_no_max_shift": ("double e = exp(s[t] - L);\n    const uint16_t* row", "double e = exp(s[t]);\n    const uint16_t* row"),
    "attn_lse_without_max": ("return L + log(sum);", "return log(sum);"),
    "attn_last_range_short": ("b = a + chunk < T ? a + chunk : T;", "b = a + chunk < T ? a + chunk : T - 1;"),
    "f64_bf16_ties_up": ("r = fmod(lo, 2.0) == 0.0 ? lo * step : (lo + 1.0) * step;", "r = (lo + 1.0) * step;"),
    "f64_bf16_one_bit_short": ("int se = e - 8;", "int se = e - 7;"),
    "qscale_ignores_q_pe": ("for (size_t i = 0; i < n_pe; ++i) {", "for (size_t i = 0; i < 0; ++i) {"),
    "qscale_signed_acc": ("float a = fabsf(acc[i]);", "float a = acc[i];"),
    "qscale_signed_q_pe": ("float a = fabsf(bf16_to_f32(q_pe[i]));", "float a = bf16_to_f32(q_pe[i]);"),
    "qscale_no_zero_guard": ("return amax == 0.0f ? 1.0f : amax / 448.0f;", "return amax / 448.0f;"),
    "qscale_divisor_480": ("return amax == 0.0f ? 1.0f : amax / 448.0f;", "return amax == 0.0f ? 1.0f : amax / 480.0f;"),
}


@pytest.mark.parametrize("name", sorted(MUTANTS))
def test_planted_mistake_is_caught(name, tmp_path):
    old, new = MUTANTS[name]
    src = oracle.SRC.read_text()
    assert src.count(old) == 1, f"mutation anchor for {name} not found exactly once"
    msrc = tmp_path / f"mutant_{name}.c"
    msrc.write_text(src.replace(old, new))
    lib = oracle.build(out=tmp_path / f"libmutant_{name}.so", src=msrc)
    failed = []
    for check in pins.ALL_CHECKS:
        try:
            check(lib=lib)
        except AssertionError:
            failed.append(check.__name__)
            break
    assert failed, f"no pin catches the planted mistake {name}"
