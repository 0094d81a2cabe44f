"""Plant plausible mistakes in a copy of the oracle's C source (on the CPU)
and check that the pin suite catches every one of them."""
import os
import shutil
import subprocess
import sys

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
SRC = os.path.join(ROOT, "oracle", "tbe_oracle.c")

# (name, original text, planted text)
MUTANTS = [
    ("forward_drops_sample_weight", "double sj = psw ? (double)psw[j] : 1.0;", "double sj = 1.0;"),
    ("backward_drops_sample_weight", "double s = sorted_psw ? (double)sorted_psw[k] : 1.0;",
     "double s = 1.0;"),
    ("adagrad_sign", "w0 - lr * g[d] / denom", "w0 + lr * g[d] / denom"),
    ("adagrad_sum_not_mean", "+ sumsq / D;", "+ sumsq;"),
    ("adagrad_eps_inside_root", "sqrt(m1) + eps", "sqrt(m1 + eps)"),
    ("adagrad_old_state", "double denom = sqrt(m1) + eps;",
     "double denom = sqrt((double)m_data[r] + 1e-30) + eps;"),
    ("grad_row_transposed", "grad + (b * T + t) * D", "grad + (t * B + b) * D"),
    ("sort_ties_reversed", "return x->pos < y->pos ? -1 : 1;", "return x->pos < y->pos ? 1 : -1;"),
    ("route_threshold_inclusive", "if (sl < S) {", "if (sl <= S) {"),
    ("route_chunk_stride", "a += C)", "a += C + 1)"),
    ("linearize_no_table_offset", "keys[j] = (int32_t)(first_row + indices[j]);",
     "keys[j] = (int32_t)(indices[j]);"),
    ("forward_layout_transposed", "out + ((int64_t)b * T + t) * D", "out + ((int64_t)t * B + b) * D"),
    ("bf16_rounding_width", "round_to_format(x, 8, -126", "round_to_format(x, 9, -126"),
    ("half_decode_bias", "exp - 25)", "exp - 24)"),
    ("histogram_sets_not_counts", "H[bag * E + indices[j]] += 1;", "H[bag * E + indices[j]] = 1;"),
    ("rle_last_offset", "run_offsets[U] = (int32_t)N;", "run_offsets[U] = (int32_t)N - (N > 0);"),
    ("backward_adds_bag_weight_squared", "g[d] += s * (double)row[d];", "g[d] += s * s * (double)row[d];"),
]


@pytest.mark.slow
@pytest.mark.parametrize("name,orig,planted", MUTANTS, ids=[m[0] for m in MUTANTS])
def test_pins_catch_planted_mistake(tmp_path, name, orig, planted):
    src = open(SRC).read()
    assert src.count(orig) == 1, f"mutation site for {name} not unique/found"
    mut = tmp_path / "mutant.c"
    mut.write_text(src.replace(orig, planted))
    so = tmp_path / "mutant.so"
    subprocess.check_call(["gcc", "-std=c11", "-O2", "-fPIC", "-shared", "-ffp-contract=off",
                           "-o", str(so), str(mut), "-lm"])
    env = dict(os.environ, TBE_ORACLE_LIB=str(so))
    r = subprocess.run([sys.executable, "-m", "pytest", "-x", "-q", "-p", "no:cacheprovider",
                        os.path.join(ROOT, "tests", "test_oracle_pins.py")],
                       cwd=ROOT, env=env, capture_output=True, text=True, timeout=600)
    assert r.returncode != 0, f"planted mistake {name} survived the pins:\n{r.stdout[-2000:]}"
