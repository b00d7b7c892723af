/*
 * Plain fp64 CPU oracle: declarations.  TEST INFRASTRUCTURE ONLY (tests,
 * smoke check and the benchmark's CPU-baseline leg).  Shares nothing with the
 * HIP library.  All arrays are host memory owned by the caller, row-major and
 * contiguous.  Definitions and their sources are documented in oracle.c.
 */
#ifndef TEA_ORACLE_H
#define TEA_ORACLE_H

#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

/* Two-pass safe softmax of rows of fp32 logits: y [rows, cols] (nullable),
 * m [rows] (natural units), l [rows] = sum exp(x - m). */
void oracle_softmax_rows(const float* x, int64_t rows, int64_t cols, double* y, double* m, double* l);
void oracle_softmax_f64(const double* x, int64_t n, double* y, double* m, double* l);

/* Naive sum exp(x); also that sum times exp(-max x); finite flag. */
void oracle_naive_normaliser(const double* x, int64_t n, double* sum_exp, double* rel_to_max, int* finite);

/* Online normaliser recurrence over contiguous blocks (see oracle.c for the
 * variants).  Traces are [number of blocks]; they and the scalar outputs are
 * nullable.  Returns the block count. */
int64_t oracle_online_trace(const double* x, int64_t n, int64_t block, int variant, double* m_trace,
                            double* l_trace, double* c_trace, int64_t* rescales, double* m_final,
                            double* l_final);

/* The recurrence with the output accumulator, for one query row. */
void oracle_online_attention_row(const double* s, const double* V, int64_t n, int64_t D, int64_t block,
                                 int variant, double* o, double* m_out, double* l_out);

/* Attention from the definition for the listed flat rows (all when NULL). */
void oracle_attention_rows(const float* Q, const float* K, const float* V, int64_t B, int64_t H, int64_t Sq,
                           int64_t Sk, int64_t D, double scale, int causal, const int64_t* rows, int64_t nrows,
                           double* O, double* lse);

/* Partial state (m, l, unnormalised O) of one set of scores. */
void oracle_partial(const double* s, const double* V, int64_t n, int64_t D, double* m_out, double* l_out,
                    double* O);

/* Pairwise combine of two partial states; output may alias an input. */
void oracle_combine(double m1, double l1, const double* O1, double m2, double l2, const double* O2, int64_t D,
                    double* m_out, double* l_out, double* O);

/* Merged state of S partials per row, written out directly. */
void oracle_merge_direct(const double* m, const double* l, const double* O, int64_t N, int64_t S, int64_t D,
                         double* m_out, double* l_out, double* O_out);

int oracle_abi_version(void);
int oracle_num_threads(void);
int oracle_set_num_threads(int n);

#ifdef __cplusplus
}
#endif

#endif
