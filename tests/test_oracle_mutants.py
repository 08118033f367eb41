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
