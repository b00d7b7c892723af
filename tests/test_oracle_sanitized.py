"""The C oracle under AddressSanitizer and UndefinedBehaviorSanitizer (host
code only): a small driver calls every exported function on small inputs,
including empty sets, -inf rows, masked and ragged attention rows and empty
partials, and must exit cleanly with no sanitizer report."""
import os
import shutil
import subprocess

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
ORACLE = os.path.join(ROOT, "oracle")

DRIVER = r"""
#include <math.h>
#include <stdio.h>
#include <stdlib.h>
#include "oracle.h"

int main(void)
{
    /* row softmax: a plain row, an all -inf row, a row with a huge spread */
    float x[3 * 5] = {0.5f, -1.0f, 2.0f, 0.0f, 3.0f,
                      -INFINITY, -INFINITY, -INFINITY, -INFINITY, -INFINITY,
                      1000.0f, -1000.0f, 0.0f, 999.0f, -INFINITY};
    double y[15], m[3], l[3];
    oracle_softmax_rows(x, 3, 5, y, m, l);
    oracle_softmax_rows(x, 3, 5, NULL, m, l);
    double xd[7] = {1, 2, 3, -INFINITY, 0.25, 7, -2};
    double yd[7], md, ld, se, rel;
    int fin;
    oracle_softmax_f64(xd, 7, yd, &md, &ld);
    oracle_naive_normaliser(xd, 7, &se, &rel, &fin);
    oracle_naive_normaliser(xd, 0, &se, &rel, &fin);

    /* online traces: every variant, blocks that do and do not divide n */
    double mt[8], lt[8], ct[8], mf, lf;
    int64_t resc;
    int variants[] = {0, 1, 2, 3, 10, 11, 12};
    for (int v = 0; v < 7; ++v)
        for (int64_t b = 1; b <= 8; b *= 2)
            oracle_online_trace(xd, 7, b, variants[v], mt, lt, ct, &resc, &mf, &lf);
    oracle_online_trace(xd, 7, 3, 0, NULL, NULL, NULL, NULL, &mf, &lf);

    /* the recurrence with an accumulator */
    double V[7 * 3], o[3], mo, lo;
    for (int i = 0; i < 21; ++i) V[i] = 0.1 * i - 1.0;
    int avar[] = {0, 10, 11, 12, 20, 21};
    for (int v = 0; v < 6; ++v) oracle_online_attention_row(xd, V, 7, 3, 2, avar[v], o, &mo, &lo);

    /* attention from the definition: causal and not, all rows and a list */
    enum { B = 1, H = 2, S = 6, D = 3 };
    float Q[B * H * S * D], K[B * H * S * D], Vf[B * H * S * D];
    for (int i = 0; i < B * H * S * D; ++i) {
        Q[i] = (float)((i * 7) % 5) * 0.3f - 0.5f;
        K[i] = (float)((i * 3) % 7) * 0.2f - 0.6f;
        Vf[i] = (float)(i % 4) - 1.5f;
    }
    double O[B * H * S * D], lse[B * H * S];
    oracle_attention_rows(Q, K, Vf, B, H, S, S, D, 0.5, 0, NULL, 0, O, lse);
    oracle_attention_rows(Q, K, Vf, B, H, S, S, D, 0.5, 1, NULL, 0, O, lse);
    int64_t rows[3] = {0, 5, 11};
    double O3[3 * D], l3[3];
    oracle_attention_rows(Q, K, Vf, B, H, S, S, D, 0.5, 1, rows, 3, O3, l3);
    oracle_attention_rows(Q, K, Vf, B, H, S, 4, D, 0.5, 0, rows, 3, O3, l3);

    /* partials, combine (with the empty state) and the direct merge */
    double pm, pl, pO[3], em = -INFINITY, el = 0.0, eO[3] = {0, 0, 0};
    oracle_partial(xd, V, 7, 3, &pm, &pl, pO);
    oracle_partial(xd, V, 0, 3, &em, &el, eO);
    double cm, cl, cO[3];
    oracle_combine(pm, pl, pO, em, el, eO, 3, &cm, &cl, cO);
    oracle_combine(em, el, eO, em, el, eO, 3, &cm, &cl, cO);
    oracle_combine(pm, pl, pO, pm, pl, pO, 3, &pm, &pl, pO); /* aliasing output */
    double mm[2 * 3] = {1.0, -INFINITY, 0.5, -INFINITY, -INFINITY, -INFINITY};
    double ll[2 * 3] = {2.0, 0.0, 1.0, 0.0, 0.0, 0.0};
    double OO[2 * 3 * 3];
    for (int i = 0; i < 18; ++i) OO[i] = (i < 9) ? 0.5 * i : 0.0;
    double mout[2], lout[2], Oout[2 * 3];
    oracle_merge_direct(mm, ll, OO, 2, 3, 3, mout, lout, Oout);

    printf("ok %d %d\n", oracle_abi_version(), oracle_num_threads() > 0);
    return 0;
}
"""


@pytest.mark.skipif(shutil.which("gcc") is None, reason="gcc not available")
def test_oracle_under_asan_and_ubsan(tmp_path):
    drv = tmp_path / "driver.c"
    drv.write_text(DRIVER)
    exe = tmp_path / "oracle_sanitized"
    cmd = ["gcc", "-O1", "-g", "-std=c11", "-fopenmp", "-ffp-contract=off", "-fno-fast-math",
           "-fsanitize=address,undefined", "-fno-sanitize-recover=all", "-fno-omit-frame-pointer",
           "-I", ORACLE, os.path.join(ORACLE, "oracle.c"), str(drv), "-o", str(exe), "-lm"]
    probe = subprocess.run(["gcc", "-fsanitize=address,undefined", "-x", "c", "-", "-o", str(tmp_path / "p")],
                           input="int main(void){return 0;}", text=True, capture_output=True)
    if probe.returncode != 0:
        pytest.skip("this gcc has no sanitizer runtime")
    subprocess.run(cmd, check=True, capture_output=True, text=True)
    env = dict(os.environ, ASAN_OPTIONS="detect_leaks=0:abort_on_error=0", UBSAN_OPTIONS="print_stacktrace=1",
               OMP_NUM_THREADS="2")
    r = subprocess.run([str(exe)], capture_output=True, text=True, env=env, timeout=120)
    assert r.returncode == 0, r.stdout + r.stderr
    assert r.stdout.startswith("ok "), r.stdout + r.stderr
    assert "runtime error" not in r.stderr and "AddressSanitizer" not in r.stderr, r.stderr
