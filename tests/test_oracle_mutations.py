"""Planted-mistake check of the oracle pins (CPU only).

Each case below plants one plausible mistake in a copy of oracle/oracle.c
(a wrong constant, a swapped nibble order, a tie broken the wrong way, an
off-by-one, a dropped weight, a wrong group index, ...), builds it into a
scratch library and runs the oracle pins against it: every mutant must fail
at least one pin.  The real oracle is never modified.

Not covered on purpose: changing the fp32 accumulation order of combine
moves results by about one fp32 ulp, below the resolution of any pin the
pages allow (they fix fp32 and a fixed slot order, not a printed value).
"""

import os
import subprocess
import sys

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
PINS = ["tests/test_oracle_formats.py", "tests/test_oracle_layout.py",
        "tests/test_oracle_payload.py", "tests/test_oracle_nvfp4.py", "tests/test_oracle_fp8.py",
        "tests/test_oracle_routing_map.py", "tests/test_oracle_combine_nvfp4.py"]

MUTANTS = {
    "global_scale_448": ("2688.0f / rowmax", "448.0f / rowmax"),
    "nibble_order": ("(uint8_t)(code[2 * j] | (code[2 * j + 1] << 4))",
                     "(uint8_t)(code[2 * j + 1] | (code[2 * j] << 4))"),
    "block_scale_div4": ("float d = bmax / 6.0f;", "float d = bmax / 4.0f;"),
    "e2m1_tie_odd": ("(err == best_err && (c & 1) == 0)) {\n            best = c;\n            best_err = err;\n"
                     "        }\n    }\n    return (uint8_t)(best | (signbit",
                     "(err == best_err && (c & 1) == 1)) {\n            best = c;\n            best_err = err;\n"
                     "        }\n    }\n    return (uint8_t)(best | (signbit"),
    "e4m3_tie_odd": ("(err == best_err && (c & 1) == 0)) {\n            best = c;\n            best_err = err;\n"
                     "        }\n    }\n    return (uint8_t)best;",
                     "(err == best_err && (c & 1) == 1)) {\n            best = c;\n            best_err = err;\n"
                     "        }\n    }\n    return (uint8_t)best;"),
    "e4m3_subnormal_exp": ("if (e == 0) v = ldexpf((float)m, -9);", "if (e == 0) v = ldexpf((float)m, -10);"),
    "rowscale_formula": ("*rowscale = orc_bf16_rne(1.0f / g);",
                         "*rowscale = orc_bf16_rne(rowmax / 2688.0f + 1e-3f * rowmax);"),
    "sign_of_negative_zero": ("return (uint8_t)(best | (signbit(v) ? 8 : 0));",
                              "return (uint8_t)(best | (v < 0.0f ? 8 : 0));"),
    "inverse_scale": ("float inv = g / sq;", "float inv = 1.0f / sq * g * 1.0001f;"),
    "block_max": ("if (a > bmax) bmax = a;", "if (i == 0) bmax = a;"),
    "align_up": ("return ((count + multiple - 1) / multiple) * multiple;",
                 "return ((count + multiple) / multiple) * multiple;"),
    "segment_of_expert": ("return (e / E_loc) * G + c->shared + (e % E_loc);",
                          "return (e % c->S) * G + c->shared + (e / c->S);"),
    "shared_group": ("return c->src_seg * G + 0;", "return c->src_seg * G + 1;"),
    "capacity_off_by_one": ("if (c->C > 0 && pos >= c->C) { dropped = 1; continue; }",
                            "if (c->C > 0 && pos > c->C) { dropped = 1; continue; }"),
    "bad_id_flag": ("if (e < 0 || e >= c->E) { *bad = 1; return -1; }",
                    "if (e < 0 || e >= c->E) { return -1; }"),
    "pad_row_metadata": ("src_info[2 * row] = -1;", "src_info[2 * row] = 0;"),
    "combine_unweighted": ("float w = slot_weight(c, probs, t, k);\n                float v",
                           "float w = 1.0f;\n                float v"),
    "combine_bwd_weight_index": ("float w = slot_weight(c, probs, t, k);\n            for",
                                 "float w = slot_weight(c, probs, t, (k + 1) % (c->K));\n            for"),
    "probs_grad_wrong_operand": ("dot += (double)orc_bf16_to_f32(grad_y[(int64_t)t * c->H + h]) *\n                           (double)orc_bf16_to_f32(out[(int64_t)row * c->H + h]);",
                                 "dot += (double)orc_bf16_to_f32(grad_y[(int64_t)t * c->H + h]) *\n                           (double)orc_bf16_to_f32(out[(int64_t)t * c->H + h]);"),
    "fp8_scale_formula": ("scales[b] = amax / 448.0f;", "scales[b] = amax / 447.0f;"),
    "fp8_inverse_scale": ("float inv = 448.0f / amax;", "float inv = 480.0f / amax;"),
    "fp8_sign_dropped": ("return signbit(v) ? (uint8_t)(c | 0x80) : c;", "return c;"),
    "multihot_overwrites": ("dense_probs[(int64_t)t * c->E + e] = dense_probs[(int64_t)t * c->E + e] + probs[(int64_t)t * c->K + k];",
                            "dense_probs[(int64_t)t * c->E + e] = probs[(int64_t)t * c->K + k];"),
    "map_overflow_unflagged": ("                flags |= 8;\n", ""),
    "bf16_truncates": ("if (rem > 0x8000u) return (uint16_t)(lo + 1);",
                       "if (rem > 0x8000u) return (uint16_t)(lo);"),
    "nvfp4_combine_nibble_order": ("(h % 2 == 0) ? (uint8_t)(byte & 0x0F) : (uint8_t)(byte >> 4)",
                                   "(h % 2 == 1) ? (uint8_t)(byte & 0x0F) : (uint8_t)(byte >> 4)"),
    "nvfp4_combine_no_rowscale": ("float block_scale = orc_e4m3_decode(scales[(int64_t)row * (H / 16) + h / 16]) *\n"
                                  "                                    orc_bf16_to_f32(rowscale[row]);",
                                  "float block_scale = orc_e4m3_decode(scales[(int64_t)row * (H / 16) + h / 16]);"),
    "nvfp4_combine_scale_index": ("scales[(int64_t)row * (H / 16) + h / 16]", "scales[(int64_t)row * (H / 16) + h / 8]"),
    "nvfp4_combine_unweighted": ("float w = slot_weight(c, probs, t, k);\n                uint8_t byte",
                                 "float w = 1.0f;\n                uint8_t byte"),
    "nvfp4_combine_sign_dropped": ("float xhat = orc_e2m1_decode(code) * block_scale;",
                                   "float xhat = orc_e2m1_decode(code & 7) * block_scale;"),
}


@pytest.mark.parametrize("name", sorted(MUTANTS))
def test_pins_catch_planted_mistake(name, tmp_path):
    src = open(os.path.join(ROOT, "oracle", "oracle.c")).read()
    old, new = MUTANTS[name]
    assert src.count(old) >= 1, f"mutation site for {name} not found"
    mutated = tmp_path / "oracle_mut.c"
    mutated.write_text(src.replace(old, new, 1))
    lib = tmp_path / "liboracle_mut.so"
    subprocess.run(["gcc", "-O2", "-fno-fast-math", "-ffp-contract=off", "-shared", "-fPIC",
                    "-o", str(lib), str(mutated), "-lm"], check=True)
    env = dict(os.environ, EPX_ORACLE_LIB_OVERRIDE=str(lib))
    r = subprocess.run([sys.executable, "-m", "pytest", "-x", "-q", "-p", "no:cacheprovider",
                        "-m", "not gpu", *PINS], cwd=ROOT, env=env, capture_output=True, text=True)
    assert r.returncode == 1, f"mutant {name} passed every pin:\n{r.stdout[-2000:]}"
