/*
 * Plain fp64 CPU oracle for the one-pass online softmax and the attention
 * built on it.  TEST INFRASTRUCTURE ONLY: the test suite, the smoke check and
 * the CPU-baseline leg of the benchmark may load this library; the product
 * path never does.  It shares no code, header or constant with the HIP
 * library.
 *
 * Every result here is computed from the plain definition, in double
 * precision, from the exact values the GPU receives (fp32, or bf16 widened to
 * fp32).  Nothing is blocked, fused or reordered beyond what the definition
 * states.  Sources, cited by page title and section:
 *   [OS-R]  "Online softmax" (roadmapper-2x4.pages.dev)
 *   [OS-C]  "The Online Softmax" (llm.curionode.com, Vol. XVI plate 3)
 *   [OS-M]  "Online Softmax" (metalworking.vercel.app)
 *
 * Conventions fixed where the pages are silent:
 *   - an empty set of logits (no element, or all -inf) has maximum -inf,
 *     normaliser 0 and output 0 (the identity of the merge); never NaN;
 *   - exported maxima and log-sum-exp values are in natural-log units.
 */
#include <math.h>
#include <omp.h>
#include <stddef.h>
#include <stdint.h>
#include <stdlib.h>
#include <string.h>

#include "oracle.h"

/* Neumaier-compensated running sum: keeps the normaliser accurate to a few
 * ulp of fp64 however many terms are added, so that the oracle's own rounding
 * stays far below every tolerance it is used for. */
typedef struct {
    double s, c;
} ksum;

static void ksum_add(ksum* k, double v)
{
    double t = k->s + v;
    if (fabs(k->s) >= fabs(v))
        k->c += (k->s - t) + v;
    else
        k->c += (v - t) + k->s;
    k->s = t;
}

static double ksum_get(const ksum* k) { return k->s + k->c; }

/* ---------------------------------------------------------------------------
 * O1  Two-pass safe softmax of one row ([OS-C] intro and "Terms: Safe
 * softmax"; [OS-M] "The problem").  Pass 1: m = max x.  Pass 2:
 * l = sum exp(x - m).  Then y = exp(x - m) / l.
 * ------------------------------------------------------------------------ */
static void softmax_row_f64(const double* x, int64_t n, double* y, double* m_out, double* l_out)
{
    double m = -INFINITY;
    for (int64_t i = 0; i < n; ++i)
        if (x[i] > m) m = x[i];
    if (m == -INFINITY) { /* empty set: merge identity */
        if (y)
            for (int64_t i = 0; i < n; ++i) y[i] = 0.0;
        *m_out = -INFINITY;
        *l_out = 0.0;
        return;
    }
    ksum acc = {0.0, 0.0};
    for (int64_t i = 0; i < n; ++i) ksum_add(&acc, exp(x[i] - m));
    double l = ksum_get(&acc);
    if (y)
        for (int64_t i = 0; i < n; ++i) y[i] = exp(x[i] - m) / l;
    *m_out = m;
    *l_out = l;
}

void oracle_softmax_rows(const float* x, int64_t rows, int64_t cols, double* y, double* m, double* l)
{
#pragma omp parallel
    {
        double* buf = (double*)malloc(sizeof(double) * (size_t)(cols > 0 ? cols : 1));
#pragma omp for schedule(static)
        for (int64_t r = 0; r < rows; ++r) {
            const float* xr = x + r * cols;
            for (int64_t j = 0; j < cols; ++j) buf[j] = (double)xr[j];
            softmax_row_f64(buf, cols, y ? y + r * cols : NULL, m + r, l + r);
        }
        free(buf);
    }
}

void oracle_softmax_f64(const double* x, int64_t n, double* y, double* m, double* l)
{
    softmax_row_f64(x, n, y, m, l);
}

/* ---------------------------------------------------------------------------
 * O3  The naive normaliser sum exp(x_i) with no maximum subtracted
 * ([OS-C] intro: it overflows for large logits; "Workshop": computed in
 * double, overflowing past e^709).  Also returns it relative to the true
 * maximum, sum exp(x) * exp(-max), which is what the workshop compares.
 * ------------------------------------------------------------------------ */
void oracle_naive_normaliser(const double* x, int64_t n, double* sum_exp, double* rel_to_max, int* finite)
{
    double m = -INFINITY;
    double s = 0.0;
    for (int64_t i = 0; i < n; ++i) {
        s += exp(x[i]);
        if (x[i] > m) m = x[i];
    }
    *sum_exp = s;
    *finite = isfinite(s) ? 1 : 0;
    *rel_to_max = s * exp(-m);
}

/* ---------------------------------------------------------------------------
 * O2  The online normaliser recurrence, run the way the pages state it, to
 * check their claims about it ([OS-R] "The recurrence", "Initialise
 * honestly", "Things that break"; [OS-C] intro and "One pass, exactly";
 * [OS-M] "The problem").  Not a parity reference for the GPU.
 *
 * The row is cut into contiguous blocks of `block` values in index order (the
 * last one partial).  Start from m = -inf, l = 0.  For each block:
 *     m' = max(m, max of the block)
 *     c  = exp(m - m')            the correction, 0 <= c <= 1
 *     l  = l * c + sum over the block of exp(x - m')
 *     m  = m'
 * A "rescale" is an update whose incoming m is finite and strictly below the
 * block maximum (the first non-empty block only initialises: c = 0).
 *
 * `variant` selects the pages' equivalent forms and the failure modes they
 * name, so tests can show the forms agree and the failures fail:
 *   0  natural base, l0 = 0, unconditional correction
 *   1  base two: logits pre-multiplied by log2(e), every exponential exp2
 *   2  the tutorial's start l0 = 1
 *   3  correction only when the maximum rises (else factor 1)
 *  10  FAILURE: maximum recomputed from each block, not carried forward
 *  11  FAILURE: mixed bases, logits in base two but the correction in base e
 *  12  FAILURE: no guard, so an all -inf first block gives -inf - -inf = NaN
 *  Variants 0..3 and 10..11 apply the guard of reading "empty set": while the
 *  running maximum is still -inf the exponent uses 0 in its place.
 * Traces have one entry per block; they and the scalar outputs may be NULL.
 * Returns the block count.
 * ------------------------------------------------------------------------ */
int64_t oracle_online_trace(const double* x, int64_t n, int64_t block, int variant, double* m_trace,
                            double* l_trace, double* c_trace, int64_t* rescales, double* m_final,
                            double* l_final)
{
    const double LOG2E = 1.4426950408889634074; /* log2(e) */
    int base2 = (variant == 1 || variant == 11);
    double m = -INFINITY;
    double l = (variant == 2) ? 1.0 : 0.0;
    int64_t nres = 0, k = 0;
    for (int64_t b0 = 0; b0 < n; b0 += block, ++k) {
        int64_t b1 = b0 + block < n ? b0 + block : n;
        double bmax = -INFINITY;
        for (int64_t i = b0; i < b1; ++i) {
            double t = base2 ? x[i] * LOG2E : x[i];
            if (t > bmax) bmax = t;
        }
        double mnew = (variant == 10) ? bmax : (m > bmax ? m : bmax);
        double muse = mnew;
        if (variant != 12 && muse == -INFINITY) muse = 0.0;
        if (isfinite(m) && bmax > m) ++nres;
        double c;
        if (variant == 3)
            c = (mnew > m) ? (base2 ? exp2(m - muse) : exp(m - muse)) : 1.0;
        else if (variant == 1)
            c = exp2(m - muse);
        else /* 11 deliberately takes base e here while the terms use base two */
            c = exp(m - muse);
        double s = 0.0;
        for (int64_t i = b0; i < b1; ++i) {
            double t = base2 ? x[i] * LOG2E : x[i];
            s += base2 ? exp2(t - muse) : exp(t - muse);
        }
        l = l * c + s;
        m = mnew;
        if (m_trace) m_trace[k] = base2 ? m / LOG2E : m;
        if (l_trace) l_trace[k] = l;
        if (c_trace) c_trace[k] = c;
    }
    if (rescales) *rescales = nres;
    if (m_final) *m_final = base2 ? m / LOG2E : m;
    if (l_final) *l_final = l;
    return k;
}

/* ---------------------------------------------------------------------------
 * The same recurrence carrying the output accumulator as well ([OS-R] "The
 * recurrence": acc = acc * alpha + p V; [OS-M] "The problem": O = O c + P V,
 * then O /= l after the last tile).  For one query row: scores s[n], values
 * V[n, D].  Used only to check the pages' claims and their failure modes.
 *   variant 0   correct
 *          20   FAILURE: l rescaled, acc not
 *          21   FAILURE: acc rescaled, l not
 *          10, 11, 12 as in oracle_online_trace
 * ------------------------------------------------------------------------ */
void oracle_online_attention_row(const double* s, const double* V, int64_t n, int64_t D, int64_t block,
                                 int variant, double* o, double* m_out, double* l_out)
{
    const double LOG2E = 1.4426950408889634074;
    int base2 = (variant == 11);
    double m = -INFINITY, l = 0.0;
    for (int64_t d = 0; d < D; ++d) o[d] = 0.0;
    for (int64_t b0 = 0; b0 < n; b0 += block) {
        int64_t b1 = b0 + block < n ? b0 + block : n;
        double bmax = -INFINITY;
        for (int64_t i = b0; i < b1; ++i) {
            double t = base2 ? s[i] * LOG2E : s[i];
            if (t > bmax) bmax = t;
        }
        double mnew = (variant == 10) ? bmax : (m > bmax ? m : bmax);
        double muse = mnew;
        if (variant != 12 && muse == -INFINITY) muse = 0.0;
        double c = exp(m - muse); /* base e in every variant: wrong for 11 */
        double lsum = 0.0;
        double scale_l = (variant == 21) ? 1.0 : c;
        double scale_o = (variant == 20) ? 1.0 : c;
        for (int64_t d = 0; d < D; ++d) o[d] *= scale_o;
        for (int64_t i = b0; i < b1; ++i) {
            double t = base2 ? s[i] * LOG2E : s[i];
            double p = base2 ? exp2(t - muse) : exp(t - muse);
            lsum += p;
            for (int64_t d = 0; d < D; ++d) o[d] += p * V[i * D + d];
        }
        l = l * scale_l + lsum;
        m = mnew;
    }
    for (int64_t d = 0; d < D; ++d) o[d] = (l == 0.0) ? 0.0 : o[d] / l;
    *m_out = base2 ? m / LOG2E : m;
    *l_out = l;
}

/* ---------------------------------------------------------------------------
 * O4  Attention from its definition, one query row at a time ([OS-C] "One
 * pass, exactly": attention's output is a softmax-weighted sum of value
 * vectors; [OS-M] intro and "The problem"):
 *     s_j  = scale * sum_d Q[i,d] K[j,d]      for every visible key j
 *     O[i] = sum_j softmax(s)_j V[j]          (two-pass safe softmax, O1)
 *     lse  = m + ln l
 * Causal visibility: key j is visible to query i iff j <= i.  A query with
 * no visible key gets O = 0 and lse = -inf.  Tensors are [B, H, S, D]
 * contiguous.  `rows` lists flat (b*H + h)*Sq + i indices to compute (all
 * when NULL); O is [nrows, D], lse is [nrows] (nullable).
 * ------------------------------------------------------------------------ */
void oracle_attention_rows(const float* Q, const float* K, const float* V, int64_t B, int64_t H, int64_t Sq,
                           int64_t Sk, int64_t D, double scale, int causal, const int64_t* rows, int64_t nrows,
                           double* O, double* lse)
{
    if (!rows) nrows = B * H * Sq;
    (void)B;
#pragma omp parallel
    {
        double* s = (double*)malloc(sizeof(double) * (size_t)(Sk > 0 ? Sk : 1));
        double* p = (double*)malloc(sizeof(double) * (size_t)(Sk > 0 ? Sk : 1));
        double* acc = (double*)malloc(sizeof(double) * (size_t)D);
#pragma omp for schedule(dynamic, 4)
        for (int64_t r = 0; r < nrows; ++r) {
            int64_t flat = rows ? rows[r] : r;
            int64_t bh = flat / Sq, i = flat % Sq;
            const float* q = Q + flat * D;
            const float* k = K + bh * Sk * D;
            const float* v = V + bh * Sk * D;
            int64_t nvis = causal ? (i + 1 < Sk ? i + 1 : Sk) : Sk;
            for (int64_t j = 0; j < nvis; ++j) {
                double dot = 0.0;
                for (int64_t d = 0; d < D; ++d) dot += (double)q[d] * (double)k[j * D + d];
                s[j] = scale * dot;
            }
            double m, l;
            softmax_row_f64(s, nvis, p, &m, &l);
            for (int64_t d = 0; d < D; ++d) acc[d] = 0.0;
            for (int64_t j = 0; j < nvis; ++j)
                for (int64_t d = 0; d < D; ++d) acc[d] += p[j] * (double)v[j * D + d];
            for (int64_t d = 0; d < D; ++d) O[r * D + d] = acc[d];
            if (lse) lse[r] = (l > 0.0) ? m + log(l) : -INFINITY;
        }
        free(s);
        free(p);
        free(acc);
    }
}

/* ---------------------------------------------------------------------------
 * Partial softmax state of a set of scores, as the pages' merge consumes it
 * ([OS-C] "One pass, exactly": partial results (m, l) that can be merged;
 * [OS-M] "Recognition guide": partial softmaxes merged with the correction).
 * For scores s[n] and values V[n, D]:
 *     m = max s,  l = sum exp(s - m),  O = sum exp(s - m) V   (unnormalised)
 * The empty set gives (-inf, 0, 0).
 * ------------------------------------------------------------------------ */
void oracle_partial(const double* s, const double* V, int64_t n, int64_t D, double* m_out, double* l_out,
                    double* O)
{
    double m = -INFINITY;
    for (int64_t i = 0; i < n; ++i)
        if (s[i] > m) m = s[i];
    for (int64_t d = 0; d < D; ++d) O[d] = 0.0;
    if (m == -INFINITY) {
        *m_out = -INFINITY;
        *l_out = 0.0;
        return;
    }
    ksum acc = {0.0, 0.0};
    for (int64_t i = 0; i < n; ++i) {
        double p = exp(s[i] - m);
        ksum_add(&acc, p);
        for (int64_t d = 0; d < D; ++d) O[d] += p * V[i * D + d];
    }
    *m_out = m;
    *l_out = ksum_get(&acc);
}

/* ---------------------------------------------------------------------------
 * O6  The pairwise combine of two partial states ([OS-C] "One pass,
 * exactly": the rescaling identity written for pairs of partial results):
 *     m = max(m1, m2),  a_i = exp(m_i - m)  (0 when m_i = -inf)
 *     l = a1 l1 + a2 l2,  O = a1 O1 + a2 O2
 * (-inf, 0, 0) is its identity.  Output may alias either input.
 * ------------------------------------------------------------------------ */
void oracle_combine(double m1, double l1, const double* O1, double m2, double l2, const double* O2, int64_t D,
                    double* m_out, double* l_out, double* O)
{
    double m = m1 > m2 ? m1 : m2;
    double a1 = 0.0, a2 = 0.0;
    if (m != -INFINITY) {
        a1 = (m1 == -INFINITY) ? 0.0 : exp(m1 - m);
        a2 = (m2 == -INFINITY) ? 0.0 : exp(m2 - m);
    }
    for (int64_t d = 0; d < D; ++d) O[d] = a1 * O1[d] + a2 * O2[d];
    *l_out = a1 * l1 + a2 * l2;
    *m_out = m;
}

/* The merged state of S partials written out directly, with no tree:
 *     M = max_s m_s,  l = sum_s l_s exp(m_s - M),  O = sum_s O_s exp(m_s - M)
 * which is what any order or tree of pairwise combines reaches in exact
 * arithmetic.  Inputs [N, S] and [N, S, D]; outputs [N], [N] and [N, D]
 * (O unnormalised). */
void oracle_merge_direct(const double* m, const double* l, const double* O, int64_t N, int64_t S, int64_t D,
                         double* m_out, double* l_out, double* O_out)
{
#pragma omp parallel for schedule(static)
    for (int64_t n = 0; n < N; ++n) {
        double M = -INFINITY;
        for (int64_t s = 0; s < S; ++s)
            if (m[n * S + s] > M) M = m[n * S + s];
        double* o = O_out + n * D;
        for (int64_t d = 0; d < D; ++d) o[d] = 0.0;
        ksum acc = {0.0, 0.0};
        if (M != -INFINITY) {
            for (int64_t s = 0; s < S; ++s) {
                double ms = m[n * S + s];
                if (ms == -INFINITY) continue;
                double a = exp(ms - M);
                ksum_add(&acc, a * l[n * S + s]);
                for (int64_t d = 0; d < D; ++d) o[d] += a * O[(n * S + s) * D + d];
            }
        }
        m_out[n] = M;
        l_out[n] = ksum_get(&acc);
    }
}

int oracle_abi_version(void) { return 1; }

/* Threads the oracle's OpenMP loops use. */
int oracle_num_threads(void)
{
    int n = 1;
#pragma omp parallel
    {
#pragma omp single
        n = omp_get_num_threads();
    }
    return n;
}

/* Run the oracle's OpenMP loops on n threads (n >= 1); used to time it on
 * one core.  Returns the previous count. */
int oracle_set_num_threads(int n)
{
    int prev = oracle_num_threads();
    if (n >= 1) omp_set_num_threads(n);
    return prev;
}
