"""The pins catch plausible mistakes: each mutant copy of oracle.c must fail at least one.

CPU only.  Every mutant is a one-place edit of a copy of oracle/oracle.c compiled into a
temporary directory (the real oracle is never modified).  Each edit keeps every memory
access in bounds.
"""

import os

import pytest

import oracle
from oracle import oracle as oracle_mod

from .oracle_pins import ALL_PINS, Orc

SRC = os.path.join(os.path.dirname(oracle_mod.__file__), "oracle.c")

# (name, text to find, replacement) -- each text must occur exactly once in oracle.c
MUTANTS = [
    ("scale_dropped",
     "const float s = alpha[i] / (float)ranks[i];\n            for (int32_t c = 0; c < d_out; ++c) yrow[c] += s * d[c];",
     "const float s = 1.0f;\n            for (int32_t c = 0; c < d_out; ++c) yrow[c] += s * d[c];"),
    ("scale_by_r_max",
     "const float s = alpha[i] / (float)ranks[i];\n            for (int32_t c = 0; c < d_out; ++c) yrow[c] += s * d[c];",
     "const float s = alpha[i] / (float)r_max;\n            for (int32_t c = 0; c < d_out; ++c) yrow[c] += s * d[c];"),
    ("delta_sign",
     "(float)ranks[i];\n            for (int32_t c = 0; c < d_out; ++c) yrow[c] += s * d[c];",
     "(float)ranks[i];\n            for (int32_t c = 0; c < d_out; ++c) yrow[c] -= s * d[c];"),
    ("expand_step_unscaled",
     "float *yrow = y + (size_t)m * d_out;\n            for (int32_t c = 0; c < d_out; ++c) yrow[c] += s * d[c];",
     "float *yrow = y + (size_t)m * d_out;\n            for (int32_t c = 0; c < d_out; ++c) yrow[c] += d[c];"),
    ("shrink_step_wrong_row",
     "const float xv = x[(size_t)m * d_in + k];",
     "const float xv = x[(size_t)((m + 1) % M) * d_in + k];"),
    ("B_transposed",
     "const float *brow = B + ((size_t)i * r_max + j) * d_out;\n                for (int32_t c = 0; c < d_out; ++c) d[c] += tj * brow[c];\n            }\n\n            /* * alpha",
     "for (int32_t c = 0; c < d_out; ++c) d[c] += tj * B[(size_t)i * r_max * d_out + ((size_t)c * r_max + j) % ((size_t)r_max * d_out)];\n            }\n\n            /* * alpha"),
    ("A_other_adapter",
     "const float *arow = A + ((size_t)i * d_in + k) * r_max;\n                for (int32_t j = 0; j < r_max; ++j) t[j] += xv * arow[j];\n            }\n\n            /* (x A_i) B_i */",
     "const float *arow = A + ((size_t)((i + 1) % n_adapters) * d_in + k) * r_max;\n                for (int32_t j = 0; j < r_max; ++j) t[j] += xv * arow[j];\n            }\n\n            /* (x A_i) B_i */"),
    ("first_k_dropped",
     "for (int32_t k = 0; k < d_in; ++k) {\n                const float xv = xrow[k];\n                const float *wrow",
     "for (int32_t k = 1; k < d_in; ++k) {\n                const float xv = xrow[k];\n                const float *wrow"),
    ("last_rank_col_dropped",
     "const float *brow = B + ((size_t)i * r_max + j) * d_out;\n                for (int32_t c = 0; c < d_out; ++c) d[c] += tj * brow[c];\n            }\n\n            /* * alpha",
     "const float *brow = B + ((size_t)i * r_max + j) * d_out;\n                if (j + 1 < r_max || r_max == 1) for (int32_t c = 0; c < d_out; ++c) d[c] += tj * brow[c];\n            }\n\n            /* * alpha"),
    ("base_dropped_on_lora_rows",
     "/* x A_i */",
     "for (int32_t c = 0; c < d_out; ++c) yrow[c] = 0.0f;\n            /* x A_i */"),
    ("W_transposed_read",
     "const float *wrow = W + (size_t)k * d_out;\n                for (int32_t c = 0; c < d_out; ++c) yrow[c] += xv * wrow[c];",
     "for (int32_t c = 0; c < d_out; ++c) yrow[c] += xv * W[((size_t)c * d_in + k) % ((size_t)d_in * d_out)];"),
    ("segments_unstable",
     "for (int32_t m = 0; m < M; ++m) {\n        if (ids[m] >= 0) perm[cursor[ids[m]]++] = m;",
     "for (int32_t m = M - 1; m >= 0; --m) {\n        if (ids[m] >= 0) perm[cursor[ids[m]]++] = m;"),
    ("fp8_bias_8",
     "ldexpf(1.0f + (float)m / 8.0f, e - 7)",
     "ldexpf(1.0f + (float)m / 8.0f, e - 8)"),
    ("fp8_subnormal_as_normal",
     "e == 0 ? ldexpf((float)m, -9)",
     "e == 0 ? ldexpf(1.0f + (float)m / 8.0f, -7)"),
    ("fp8_sign_dropped",
     "return sign ? -v : v;",
     "return v;"),
    ("fp8_scale_dropped",
     "for (int32_t c = 0; c < d_out; ++c) yrow[c] = w_scale[c] * yrow[c];",
     "for (int32_t c = 0; c < d_out; ++c) yrow[c] = yrow[c];"),
    ("fp8_W8_transposed_read",
     "Wd[(size_t)k * d_out + c] = oracle_fp8_e4m3_decode(W8[(size_t)c * d_in + k]);",
     "Wd[(size_t)k * d_out + c] = oracle_fp8_e4m3_decode(W8[(size_t)k * d_out + c]);"),
    ("fp8_delta_dropped",
     "for (int32_t c = 0; c < d_out; ++c) yrow[c] += sc * d[c];",
     "for (int32_t c = 0; c < d_out; ++c) yrow[c] += 0.0f * d[c];"),
    ("moe_wrong_expert",
     "const float *We = W + (size_t)e * d_in * d_out;",
     "const float *We = W + (size_t)((e + 1) % n_experts) * d_in * d_out;"),
    ("moe_adapter_expert_swapped",
     "const float *Aie = A + ((size_t)i * n_experts + e) * d_in * r_max;",
     "const float *Aie = A + ((size_t)e * n_adapters + i) % ((size_t)n_adapters * n_experts) * d_in * r_max;"),
    ("moe_weight_dropped",
     "for (int32_t c = 0; c < d_out; ++c) out[c] = wt * out[c];",
     "for (int32_t c = 0; c < d_out; ++c) out[c] = out[c];"),
    ("moe_empty_slot_gets_expert0",
     "if (e < 0) continue; /* empty slot */",
     "if (e < 0 && n_experts < 0) continue;"),
    ("moe_delta_unscaled",
     "for (int32_t c = 0; c < d_out; ++c) out[c] += sa * dq[c];",
     "for (int32_t c = 0; c < d_out; ++c) out[c] += dq[c];"),
    ("base_rows_first",
     "int32_t base_pos = n_lora_rows;",
     "int32_t base_pos = n_lora_rows; for (int32_t i = 0; i < n_adapters; ++i) { offsets[i] += M - n_lora_rows; cursor[i] += M - n_lora_rows; } base_pos = 0;"),
]


def _mutant_source(find, repl):
    with open(SRC) as f:
        text = f.read()
    assert text.count(find) == 1, f"mutation anchor not unique/present: {find[:60]!r}"
    return text.replace(find, repl)


@pytest.mark.parametrize("name,find,repl", MUTANTS, ids=[m[0] for m in MUTANTS])
def test_mutant_is_caught(tmp_path, name, find, repl):
    src = tmp_path / f"oracle_{name}.c"
    src.write_text(_mutant_source(find, repl))
    so = tmp_path / f"liboracle_{name}.so"
    oracle_mod.build(force=True, src=str(src), out=str(so))
    orc = Orc(oracle, oracle_mod.load_library(str(so)))
    failed = []
    for pin in ALL_PINS:
        try:
            pin(orc)
        except AssertionError:
            failed.append(pin.__name__)
    assert failed, f"mutant {name} passed every pin"
