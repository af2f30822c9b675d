"""The oracle's pins must catch plausible mistakes (CPU only).

Each case below plants one mistake in a copy of oracle/oracle.c (a dropped
term, a flipped sign, a swapped index, a missed offset, a wrong rounding),
builds it into a scratch library and runs tests/test_oracle_pins.py against
it.  The pins pass on the real oracle (that file's own run) and must fail on
every mutant here.
"""
import concurrent.futures
import os
import subprocess
import sys
import tempfile

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
SRC = os.path.join(ROOT, "oracle", "oracle.c")

MUTANTS = {
    "sum_instead_of_mean": ("ss / (double)d + (double)eps", "ss + (double)eps"),
    "eps_outside_sqrt": ("sqrt(ss / (double)d + (double)eps)", "(sqrt(ss / (double)d) + (double)eps)"),
    "weight_dropped": ("rrms * (double)w[i]", "rrms"),
    "rotation_sign_first": ("n[i] * c - n[j] * s", "n[i] * c + n[j] * s"),
    "rotation_sign_second": ("n[j] * c + n[i] * s", "n[j] * c - n[i] * s"),
    "neox_partner_swapped": ("i = p;\n            j = p + r / 2;", "i = p + r / 2;\n            j = p;"),
    "adjacent_partner_swapped": ("i = 2 * p;\n            j = 2 * p + 1;", "i = 2 * p + 1;\n            j = 2 * p;"),
    "token_base_ignored": ("int64_t t = rope->token_base + tok;", "int64_t t = tok;"),
    "plane_stride_ignored": ("(int64_t)a * rope->pos_stride + t", "(int64_t)a + t"),
    "angle_not_rounded_to_fp32": ("float theta = (float)((float)pos * rope->inv_freq[p]);",
                                  "double theta = (double)pos * rope->inv_freq[p];"),
    "axes_sections_shifted": ("if (p < end)", "if (p <= end)"),
    "imrope_residues_rotated": ("layout[3 * k + a] = a;", "layout[3 * k + (a + 1) % 3] = a;"),
    "imrope_count_from_next_axis": ("k < s[a] && 3 * k + a < period", "k < s[(a + 1) % 3] && 3 * k + a < period"),
    "imrope_t_run_short": ("k < s[a] && 3 * k + a < period", "k < s[a] - (a == 0) && 3 * k + a < period"),
    "imrope_period_without_e": ("const int32_t period = s[0] + s[1] + s[2] + s[3];",
                                "const int32_t period = s[0] + s[1] + s[2];"),
    "vit_cells_column_major": ("pos[n_tokens + n] = brow * merge + i;\n                                "
                               "pos[2 * n_tokens + n] = bcol * merge + j;",
                               "pos[n_tokens + n] = brow * merge + j;\n                                "
                               "pos[2 * n_tokens + n] = bcol * merge + i;"),
    "vit_blocks_column_major": ("for (int32_t brow = 0; brow < h / merge; ++brow)\n"
                                "                for (int32_t bcol = 0; bcol < w / merge; ++bcol)",
                                "for (int32_t bcol = 0; bcol < w / merge; ++bcol)\n"
                                "                for (int32_t brow = 0; brow < h / merge; ++brow)"),
    "vit_h_w_swapped": ("pos[n_tokens + n] = brow * merge + i;\n                                "
                        "pos[2 * n_tokens + n] = bcol * merge + j;",
                        "pos[2 * n_tokens + n] = brow * merge + i;\n                                "
                        "pos[n_tokens + n] = bcol * merge + j;"),
    "vit_frame_not_counted": ("pos[n] = t;", "pos[n] = 0;"),
    "no_contract_rounding": ("n[i] = oracle_round_bf16(n[i]);", "n[i] = n[i];"),
    "ties_away_from_zero": ("nearbyint(ldexp(v, -q))", "round(ldexp(v, -q))"),
    "truncating_bf16": ("nearbyint(ldexp(v, -q))", "trunc(ldexp(v, -q))"),
    "joint_weights_swapped": ("qw = qw_img; kw = kw_img;", "qw = qw_txt; kw = kw_txt;"),
    "joint_local_token_positions": ("rope, tau, n, q_out", "rope, tau % (tau < tokens_txt ? tokens_txt : tokens_img), n, q_out"),
    "joint_v_from_text_only": ("memcpy(v_out + dst, v,", "memcpy(v_out + dst, v_txt,"),
    "vit_plane_column_offset": ("idx = ((int64_t)a * n_tokens + n) * half_rot + off[a] + j;",
                                "idx = ((int64_t)a * n_tokens + n) * half_rot + j;"),
    "planes_read_wrong_plane": ("int64_t idx = ((int64_t)a * rope->planes_tokens + t) * half + p;",
                                "int64_t idx = ((int64_t)0 * rope->planes_tokens + t) * half + p;"),
    "vit_fused_h_w_ladders_swapped": ("inv[half_t + j] = inv_h[j];", "inv[half_t + j] = inv_w[j];"),
    "vit_fused_axes_misordered": ("rope.sections[0] = half_t;\n        rope.sections[1] = half_h;",
                                  "rope.sections[0] = half_h;\n        rope.sections[1] = half_t;"),
    "fp8_ties_away": ("double q = nearbyint(ldexp(a, 3 - k));", "double q = round(ldexp(a, 3 - k));"),
    "fp8_no_saturation": ("if (a >= 448.0)\n        return sign | 0x7E;", "if (a >= 1e300)\n        return sign | 0x7E;"),
    "fp8_subnormals_flushed": ("return sign | (uint8_t)nearbyint(ldexp(a, 9));", "return sign;"),
    "fp8_exponent_bias_off": ("(((k + 7) << 3) | ((int)q - 8))", "(((k + 8) << 3) | ((int)q - 8))"),
    "fp8_scale_multiplied": ("(float)((double)y32 / (double)scale)", "(float)((double)y32 * (double)scale)"),
    "add_norm_sum_unrounded": ("s[i] = round_out(sum, act_kind);", "s[i] = (float)sum;"),
    "add_norm_residual_ignored": ("? (double)xr[i] + (double)r[row * width + i] : (double)xr[i]",
                                  "? (double)xr[i] : (double)xr[i]"),
    "cache_written_at_token_row": ("memcpy(k_cache + slot * row, k_rot + t * row,", "memcpy(k_cache + t * row, k_rot + t * row,"),
    "cache_v_receives_k": ("memcpy(v_cache + slot * row, v + t * row,", "memcpy(v_cache + slot * row, k_rot + t * row,"),
    "cache_last_slot_dropped": ("if (slot < 0 || slot >= num_slots)\n            continue;",
                                "if (slot < 0 || slot >= num_slots - 1)\n            continue;"),
    "passthrough_skipped": ("for (int32_t i = r; i < d; ++i)\n        out[i] = round_out(n[i], out_kind);",
                            "for (int32_t i = r; i < d; ++i)\n        out[i] = 0.0f;"),
    "eager_x_rrms_not_rounded": ("const double xs = (double)round_out((double)mul32(x[i], r32), act_kind);",
                                 "const double xs = (double)mul32(x[i], r32);"),
    "eager_weight_product_not_rounded": ("u[i] = (double)round_out(xs * (double)w[i], act_kind);",
                                         "u[i] = xs * (double)w[i];"),
    "eager_rrms_not_fp32": ("(double)mul32(x[i], r32)", "(double)(float)((double)x[i] * rrms)"),
    "eager_table_not_in_activation_type": (
        "const float ct = round_out((double)(float)c, out_kind), st = round_out((double)(float)s, out_kind);",
        "const float ct = (float)c, st = (float)s;"),
    "eager_fused_multiply_add": ("out[i] = round_out((double)sub32(mul32(ni, ct), mul32(nj, st)), out_kind);",
                                 "out[i] = round_out((double)(float)((double)ni * (double)ct - "
                                 "(double)mul32(nj, st)), out_kind);"),
    "eager_rotation_sign": ("sub32(mul32(ni, ct), mul32(nj, st))", "add32(mul32(ni, ct), mul32(nj, st))"),
}


def _run_mutant(name, old, new, tmp):
    src = open(SRC).read()
    assert src.count(old) >= 1, f"mutant {name}: pattern not found in oracle.c"
    mutated = src.replace(old, new, 1)
    c_path = os.path.join(tmp, f"{name}.c")
    so_path = os.path.join(tmp, f"{name}.so")
    with open(c_path, "w") as f:
        f.write(mutated)
    subprocess.run(["gcc", "-O2", "-std=c11", "-fPIC", "-shared", "-ffp-contract=off",
                    "-I", os.path.join(ROOT, "oracle"), "-o", so_path, c_path, "-lm"],
                   check=True)
    env = dict(os.environ, ORACLE_LIB=so_path)
    r = subprocess.run([sys.executable, "-m", "pytest", "-x", "-q", "-p", "no:cacheprovider",
                        os.path.join(ROOT, "tests", "test_oracle_pins.py")],
                       cwd=ROOT, env=env, capture_output=True, text=True, timeout=300)
    return r.returncode


def test_every_planted_mistake_fails_a_pin():
    with tempfile.TemporaryDirectory() as tmp:
        with concurrent.futures.ThreadPoolExecutor(max_workers=6) as ex:
            futs = {name: ex.submit(_run_mutant, name, old, new, tmp)
                    for name, (old, new) in MUTANTS.items()}
            codes = {name: f.result() for name, f in futs.items()}
    survivors = [name for name, rc in codes.items() if rc == 0]
    assert not survivors, f"mutants not caught by any pin: {survivors}"
