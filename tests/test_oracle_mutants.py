"""Mutation test of the oracle's pins: each plausible mistake, planted in a
copy of the oracle's C source and built on the CPU, must fail at least one
pin check, while the unmodified source passes them all."""
import json
import os
import subprocess
import sys

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
SRC = os.path.join(ROOT, "oracle", "mxq_oracle.c")
BATTERY = os.path.join(ROOT, "tests", "mutant_battery.py")
CFLAGS = ["-std=c11", "-O2", "-fPIC", "-shared", "-ffp-contract=off", "-fno-fast-math"]

# (id, exact source text, replacement)
MUTANTS = [
    ("exponent_rule_floor", "if (amax <= 448.0 * ldexp(1.0, c - 127))",
     "if (amax < 256.0 * ldexp(1.0, c - 126))"),
    ("no_ftz_on_reciprocal", "    if (scale < FLT_MIN)\n        return 0.0;\n", ""),
    ("zero_block_scale_one", "    for (c = 0; c <= 254; ++c)\n        if (amax <= 448.0",
     "    if (amax == 0.0)\n        return 127;\n    for (c = 0; c <= 254; ++c)\n        if (amax <= 448.0"),
    ("scale_code_search_from_one", "    for (c = 0; c <= 254; ++c)\n        if (amax <= 448.0",
     "    for (c = 1; c <= 254; ++c)\n        if (amax <= 448.0"),
    ("ties_away_from_zero", "return nearbyint(a / spacing) * spacing;",
     "return round(a / spacing) * spacing;"),
    ("nibbles_swapped", "payload[i / 2] |= (uint8_t)(q << (4 * (i & 1)));",
     "payload[i / 2] |= (uint8_t)(q << (4 * ((i + 1) & 1)));"),
    ("swizzle_transposed", "(r % 32) * 16 + ((r % 128) / 32) * 4",
     "(r % 32) * 4 + ((r % 128) / 32) * 16"),
    ("swizzle_tiles_column_major", "((r / 128) * tiles_per_row_band + c / 4) * 512",
     "((c / 4) * ((r / 128) + 1) + r / 128) * 512"),
    ("nvfp4_multiplier_reciprocal", "m = g / sq; /* fp32 division, correctly rounded (may overflow to inf) */",
     "m = 1.0f / (sq / g);"),
    ("nvfp4_scale_divisor", "t = a / 6.0f;", "t = a / 4.0f;"),
    ("sign_of_zero_dropped", "uint8_t sign = signbit(v) ? 0x80 : 0x00;",
     "uint8_t sign = v < 0 ? 0x80 : 0x00;"),
    ("e4m3_overflow_to_nan", "return sign | 0x7E; /* saturate, never NaN */",
     "return sign | 0x7F;"),
    ("e2m1_saturates_to_4", "return sign | 0x7; /* saturate */", "return sign | 0x6;"),
    ("e4m3_subnormal_grid", "r = round_to_grid(a, -6, 3);", "r = round_to_grid(a, -7, 3);"),
    ("bf16_exponent_bias", "v = ldexp((double)(128 + m), e - 134);",
     "v = ldexp((double)(128 + m), e - 133);"),
    ("rmsnorm_mean_divisor", "den = sqrt(ss / (double)H + (double)eps);",
     "den = sqrt(ss / (double)(H - 1) + (double)eps);"),
    ("rmsnorm_eps_outside_root", "den = sqrt(ss / (double)H + (double)eps);",
     "den = sqrt(ss / (double)H) + (double)eps;"),
    ("empty_split_padded_to_128", "    return round_up(rows, 128) * round_up(sf_cols, 4);",
     "    return round_up(rows > 0 ? rows : 1, 128) * round_up(sf_cols, 4);"),
    ("split_offset_off_by_one", "for (j = 0; j < i && j < n; ++j)",
     "for (j = 0; j <= i && j < n; ++j)"),
    ("mx_element_scale_sign", "payload[i] = orc_e4m3_encode(orc_bf16_value(x[i]) * m);",
     "payload[i] = orc_e4m3_encode(orc_bf16_value(x[i]) / (m == 0.0 ? 1.0 : m) * 0.0 + orc_bf16_value(x[i]) * m * 2.0);"),
    ("residual_not_rounded",
     "uint16_t rb = orc_bf16_round(orc_bf16_value(x[t * H + j]) + orc_bf16_value(res[t * H + j]));",
     "uint16_t rb = orc_bf16_round(orc_bf16_value(x[t * H + j]));"),
    ("row_scale_uncapped", "    if (g > g_max)\n        g = g_max;\n", ""),
    ("row_scale_capped_at_flt_max", "    if (g > g_max)\n        g = g_max;\n",
     "    if (g > FLT_MAX)\n        g = FLT_MAX;\n"),
    ("row_scale_capped_at_2_100", "const float g_max = FLT_MAX / 512.0f;",
     "const float g_max = 0x1p100f;"),
    ("row_scale_lower_clamp_2_m100", "    if (g > g_max)\n        g = g_max;\n",
     "    if (g > g_max)\n        g = g_max;\n    if (g < 0x1p-100f)\n        g = 0x1p-100f;\n"),
    ("nvfp4_overflowing_multiplier_kept", "if (!(m >= FLT_MIN && m <= FLT_MAX))",
     "if (!(m >= FLT_MIN))"),
    ("nvfp4_subnormal_multiplier_kept", "if (!(m >= FLT_MIN && m <= FLT_MAX))",
     "if (!(m <= FLT_MAX))"),
    ("row_scale_zero_row_unity_dropped", "    if (amax == 0.0f)\n        return 1.0f;\n", ""),
    ("row_scale_without_e2m1_max", "g = 2688.0f / amax;", "g = 448.0f / amax;"),
    ("row_scaled_local_row_ignored",
     "scales[base + orc_sf_offset(r, c, C, layout)] = sc;",
     "scales[base + orc_sf_offset(r ? r - 1 : 0, c, C, layout)] = sc;"),
    ("split_payload_row_width_nvfp4",
     "int64_t payload_row = fmt == ORC_MXFP8 ? cols : cols / 2;\n    int64_t C;",
     "int64_t payload_row = cols / 2;\n    int64_t C;"),
    ("tensor_amax_ignores_stride", "double v = fabs(orc_bf16_value(src[r * ld + j]));",
     "double v = fabs(orc_bf16_value(src[r * cols + j]));"),
    ("tensor_amax_signed", "            double v = fabs(orc_bf16_value(src[r * ld + j]));",
     "            double v = orc_bf16_value(src[r * ld + j]);"),
]


def _run_battery(so):
    p = subprocess.run([sys.executable, BATTERY, so], capture_output=True, text=True, timeout=600)
    if p.returncode != 0:
        return None  # the build under test crashed: counts as detected
    return json.loads(p.stdout.strip().splitlines()[-1])


def _build(tmp_path, name, text):
    src = tmp_path / f"{name}.c"
    src.write_text(text)
    shutil_h = tmp_path / "mxq_oracle.h"
    if not shutil_h.exists():
        shutil_h.write_text(open(os.path.join(ROOT, "oracle", "mxq_oracle.h")).read())
    so = tmp_path / f"lib{name}.so"
    subprocess.run(["gcc", *CFLAGS, str(src), "-o", str(so), "-lm"], check=True)
    return str(so)


def test_unmutated_source_passes_every_pin(tmp_path):
    so = _build(tmp_path, "orig", open(SRC).read())
    res = _run_battery(so)
    assert res is not None and res["failed"] == [], res


@pytest.mark.parametrize("name,old,new", MUTANTS, ids=[m[0] for m in MUTANTS])
def test_mutant_is_detected(tmp_path, name, old, new):
    text = open(SRC).read()
    assert text.count(old) == 1, f"mutation site not found once: {name}"
    so = _build(tmp_path, name, text.replace(old, new))
    res = _run_battery(so)
    assert res is None or res["failed"], f"mutant {name} passed every pin"
