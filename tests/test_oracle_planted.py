"""Plant plausible mistakes in the oracle's C source, one at a time, rebuild
it on the CPU, and check that the pins in test_oracle_pins.py catch every one
of them (a dropped term, a wrong sign or index, a transposed or wrong
operand).  The oracle itself is never modified on disk."""
import os
import subprocess

import pytest

import oracle
import test_oracle_pins as pins

SRC = os.path.join(os.path.dirname(oracle.__file__), "oracle.c")

# (name, original text, planted text)
MUTANTS = [
    ("dropped scale", "s[j] = scale * dot;", "s[j] = dot;"),
    ("diagonal key hidden", "int64_t nvis = causal ? (i + 1 < Sk ? i + 1 : Sk) : Sk;",
     "int64_t nvis = causal ? (i < Sk ? i : Sk) : Sk;"),
    ("K taken for V", "acc[d] += p[j] * (double)v[j * D + d];", "acc[d] += p[j] * (double)k[j * D + d];"),
    ("K read transposed", "dot += (double)q[d] * (double)k[j * D + d];", "dot += (double)q[d] * (double)k[d * Sk + j];"),
    ("dropped dot term", "for (int64_t d = 0; d < D; ++d) dot +=", "for (int64_t d = 1; d < D; ++d) dot +="),
    ("sign of exponent", "y[i] = exp(x[i] - m) / l;", "y[i] = exp(m - x[i]) / l;"),
    ("sign of log l", "lse[r] = (l > 0.0) ? m + log(l) : -INFINITY;", "lse[r] = (l > 0.0) ? m - log(l) : -INFINITY;"),
    ("max comparison reversed", "        if (x[i] > m) m = x[i];\n    if (m == -INFINITY) {",
     "        if (x[i] < m || m == -INFINITY) m = x[i];\n    if (m == -INFINITY) {"),
    ("compensation sign", "k->c += (k->s - t) + v;", "k->c += (k->s - t) - v;"),
    ("recurrence without correction", "l = l * c + s;", "l = l + s;"),
    ("combine weight index", "O[d] = a1 * O1[d] + a2 * O2[d];", "O[d] = a1 * O1[d] + a1 * O2[d];"),
    ("merge exponent sign", "double a = exp(ms - M);", "double a = exp(M - ms);"),
    ("merge output index transposed", "o[d] += a * O[(n * S + s) * D + d];", "o[d] += a * O[(s * N + n) * D + d];"),
    ("merge output weight dropped", "o[d] += a * O[(n * S + s) * D + d];", "o[d] += O[(n * S + s) * D + d];"),
    ("merge normaliser index transposed", "ksum_add(&acc, a * l[n * S + s]);", "ksum_add(&acc, a * l[s * N + n]);"),
]

CHECKS = [
    pins.test_workshop_updates_match_printed_count,
    pins.test_online_normaliser_matches_two_pass_to_rounding,
    pins.test_closed_forms_softmax,
    pins.test_closed_forms_attention,
    lambda: pins.test_rows_sum_to_one(30.0),
    lambda: pins.test_decimal_brute_force_softmax(1000.0),
    lambda: pins.test_decimal_brute_force_attention(True),
    pins.test_torch_crosscheck_softmax,
    lambda: pins.test_torch_crosscheck_attention(False, 7, 13),
    lambda: pins.test_torch_crosscheck_attention(True, 19, 19),
    pins.test_merge_any_partition_order_tree,
    pins.test_split_kv_chunks_reach_full_decode,
    lambda: pins.test_merge_direct_output_matches_attention_of_whole_set(7),
    lambda: pins.test_merge_direct_output_matches_attention_of_whole_set(64),
]


def _first_failing_check():
    for i, chk in enumerate(CHECKS):
        try:
            chk()
        except Exception:  # an assertion, or the hypothesis wrapper reporting one
            return i
    return None


def test_unplanted_oracle_passes_every_check():
    assert _first_failing_check() is None


@pytest.mark.parametrize("name,old,new", MUTANTS, ids=[m[0] for m in MUTANTS])
def test_planted_mistake_is_caught(tmp_path, name, old, new):
    src = open(SRC).read()
    assert src.count(old) == 1, f"mutation site for '{name}' not unique"
    planted = tmp_path / "oracle_planted.c"
    planted.write_text(src.replace(old, new))
    so = tmp_path / "liboracle_planted.so"
    subprocess.run(["gcc", *oracle.CFLAGS, "-I", os.path.dirname(SRC), str(planted), "-o", str(so), "-lm"],
                   check=True)
    prev = oracle._swap_library(str(so))
    try:
        caught = _first_failing_check()
    finally:
        oracle._restore_library(prev)
    assert caught is not None, f"planted mistake '{name}' passed every pin"
