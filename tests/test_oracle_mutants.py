"""The oracle's pins must catch plausible mistakes (CPU only).

Each mutant below plants one mistake in a copy of oracle/zs_oracle.c (a
dropped term, a wrong sign, a swapped constant, a wrong index or order), builds
it with gcc into a temporary directory, and runs tests/test_oracle_pins.py
against it through the ZS_ORACLE_LIB override.  The pin suite must fail for
every mutant, and pass for the unmodified source.
"""
import os
import subprocess
import sys
import tempfile
from concurrent.futures import ThreadPoolExecutor

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
SRC = os.path.join(ROOT, "oracle", "zs_oracle.c")

MUTANTS = {
    "m_uses_c2": [("(c->b1 * m[i]) + (c->c1 * gi)", "(c->b1 * m[i]) + (c->c2 * gi)")],
    "v_drops_one_g": [("((c->c2 * gi) * gi)", "(c->c2 * gi)")],
    "mh_uses_bc2": [("float mh = mi / c->bc1;", "float mh = mi / c->bc2;")],
    "eps_inside_sqrt": [("(mh / (sqrtf(vh) + c->eps))", "(mh / sqrtf(vh + c->eps))")],
    "drops_weight_decay": [("(mh / (sqrtf(vh) + c->eps)) + (c->wd * w[i])",
                            "(mh / (sqrtf(vh) + c->eps))")],
    "decay_uses_new_m": [("(c->wd * w[i])", "(c->wd * mi)")],
    "wrong_update_sign": [("w[i] = w[i] - (c->lr * u);", "w[i] = w[i] + (c->lr * u);")],
    "sum_not_mean": [("g_out[i] = s / nd;", "g_out[i] = s;")],
    "drops_last_rank": [("for (int32_t r = 1; r < n_d; ++r)\n            s = s + or_bf16",
                         "for (int32_t r = 1; r < n_d - 1; ++r)\n            s = s + or_bf16")],
    "reverse_rank_order": [("float s = or_bf16_to_f32(slices[0][i]);",
                            "float s = or_bf16_to_f32(slices[n_d - 1][i]);"),
                           ("s = s + or_bf16_to_f32(slices[r][i]);",
                            "s = s + or_bf16_to_f32(slices[n_d - 1 - r][i]);")],
    "sqnorm_not_squared": [("uint64_t sq = M * M;", "uint64_t sq = M;")],
    "sqnorm_wrong_weight": [("big_add_shifted(L, a->lo[b], a->hi[b], 2 * (b - 1));",
                             "big_add_shifted(L, a->lo[b], a->hi[b], 2 * b);")],
    "sqnorm_drops_subnormals": [("uint32_t b = (e == 0) ? 1u : e;", "uint32_t b = e;")],
    "sqnorm_truncates": [("if (round && (sticky || (mant & 1u))) {", "if (0) {")],
    "sqnorm_ties_away": [("if (round && (sticky || (mant & 1u))) {", "if (round) {")],
    "sqnorm_drops_carry": [("if (a->lo[b] < before) a->hi[b] += 1u;", "(void)before;")],
    "clip_eps_misplaced": [("max_norm / (sqrt(Q) + 1e-6)", "max_norm / sqrt(Q) + 1e-6")],
    "clip_clamp_inverted": [("if (c > 1.0) c = 1.0;", "if (c < 1.0) c = 1.0;")],
    "clip_ignores_other_shards": [("or_clip_coef(q + other_sqnorm, h->max_grad_norm)",
                                   "or_clip_coef(q, h->max_grad_norm)")],
    "clip_not_applied": [("if (use_coef) gi = gi * coef;", "(void)use_coef;")],
    "bias_correction_t_minus_1": [("c->bc1 = (float)(1.0 - pow(h->beta1, t));",
                                   "c->bc1 = (float)(1.0 - pow(h->beta1, t + 1.0));")],
    "constant_from_float_difference": [("c->c1 = (float)(1.0 - h->beta1);",
                                        "c->c1 = 1.0f - (float)h->beta1;")],
    "pads_not_zero": [("for (int64_t i = valid_len; i < shard_len; ++i) out[i] = 0;",
                       "for (int64_t i = valid_len; i < shard_len; ++i) out[i] = 0x3F80;")],
    "bf16_ties_away": [("if (lo > 0x8000u || (lo == 0x8000u && (hi & 1u)))",
                        "if (lo >= 0x8000u)")],
    "bf16_truncates": [("        hi += 1u;\n", "        hi += 0u;\n")],
    "bf16_nan_keeps_sign": [("return (uint16_t)0x7FC0u;", "return (uint16_t)(((u >> 16) & 0x8000u) | 0x7FC0u);")],
    "layout_offset_unpadded": [("off = (int64_t)rank * S;", "off = (int64_t)rank * chunk;")],
    "layout_no_align": [("S = ((chunk + align - 1) / align) * align;", "S = chunk;")],
    "zero2_state_drops_grad": [("case 2: return 2.0 * psi + (2.0 + K) * psi / n_d;",
                                "case 2: return 2.0 * psi + K * psi / n_d;")],
    "zero3_comm_as_ddp": [("case 3: return 3.0 * psi;", "case 3: return 2.0 * psi;")],
    "f64_drops_weight_decay": [("(mh / (sqrt(vh) + h->eps) + h->weight_decay * w[i])",
                                "(mh / (sqrt(vh) + h->eps))")],
    "f64_mean_is_sum": [("g_out[i] = s / (double)n_d;", "g_out[i] = s;")],
    "f32in_wrong_rank_index": [("sum = sum + slices[r][i];", "sum = sum + slices[0][i];")],
    "f32in_sum_not_mean": [("g_out[i] = sum / ranks;", "g_out[i] = sum;")],
    "f32in_reverse_order": [("float sum = slices[0][i];", "float sum = slices[n_d - 1][i];"),
                            ("sum = sum + slices[r][i];", "sum = sum + slices[n_d - 1 - r][i];")],
    "token_weight_float_division": [("w_out[r] = (float)((double)tokens[r] / T);",
                                     "w_out[r] = (float)tokens[r] / (float)T;")],
    "token_zero_total_accepted": [("if (T == 0.0) return -2;", "")],
    "token_negative_accepted": [("if (tokens[r] < 0) return -1;", "")],
    "weighted_drops_first_weight": [("float s = w[0] * slice_value(f32in, slices[0], i);",
                                     "float s = slice_value(f32in, slices[0], i);")],
    "weighted_wrong_weight_index": [("const float p = w[r] * slice_value(f32in, slices[r], i);",
                                     "const float p = w[0] * slice_value(f32in, slices[r], i);")],
    "accumulate_sum_not_mean": [("if (j == m - 1 && m > 1) a = a / mf;", "")],
    "accumulate_reads_acc_first": [("float a = (j == 0) ? r_j[i] : acc[i] + r_j[i];",
                                    "float a = acc[i] + r_j[i];")],
    "accumulate_divides_every_step": [("if (j == m - 1 && m > 1) a = a / mf;",
                                       "if (m > 1) a = a / mf;")],
}


def _run_pins(lib_path):
    env = dict(os.environ, ZS_ORACLE_LIB=lib_path, OMP_NUM_THREADS="1")
    r = subprocess.run([sys.executable, "-m", "pytest", "-x", "-q", "-p", "no:cacheprovider",
                        os.path.join(ROOT, "tests", "test_oracle_pins.py")],
                       cwd=ROOT, env=env, capture_output=True, text=True, timeout=600)
    return r.returncode


def _build(src_text, out_dir, name):
    c_path = os.path.join(out_dir, name + ".c")
    so_path = os.path.join(out_dir, "lib" + name + ".so")
    with open(c_path, "w") as f:
        f.write(src_text)
    subprocess.run(["gcc", "-O2", "-ffp-contract=off", "-fno-fast-math", "-fPIC",
                    "-shared", "-std=c11", "-I", os.path.join(ROOT, "oracle"),
                    "-o", so_path, c_path, "-lm"], check=True)
    return so_path


def _mutate(text, edits):
    for old, new in edits:
        assert text.count(old) == 1, f"mutation anchor not unique or missing: {old!r}"
        text = text.replace(old, new)
    return text


@pytest.mark.slow
def test_every_mutant_is_caught():
    with open(SRC) as f:
        pristine = f.read()
    with tempfile.TemporaryDirectory() as d:
        base = _build(pristine, d, "pristine")
        assert _run_pins(base) == 0, "pins must pass on the unmodified oracle"
        libs = {name: _build(_mutate(pristine, edits), d, name)
                for name, edits in MUTANTS.items()}
        with ThreadPoolExecutor(max_workers=4) as ex:
            codes = dict(zip(libs, ex.map(_run_pins, libs.values())))
    survivors = [n for n, rc in codes.items() if rc == 0]
    assert not survivors, f"mutants not caught by any pin: {survivors}"
