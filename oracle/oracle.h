/*
 * oracle.h -- CPU oracle for the recurrent-state decode step of Gated DeltaNet (GDN) and
 * Kimi Delta Attention (KDA) with the state held as FP32, as uniform INT8, or in DAMP's
 * mixed layout (FP16 high-risk key rows, INT8 + per-row scale for the rest).
 *
 * TEST INFRASTRUCTURE ONLY. The test suite, the smoke check and the benchmark's CPU-baseline
 * leg are the only code allowed to load this library. It shares no source, header, table or
 * helper with the GPU library, and the GPU library never calls it.
 *
 * Sources (web pages; see oracle.c for the step-by-step citations):
 *   - "STEPQuant: When and Where Errors Matter in Delta-Rule Recurrent State Quantization",
 *     appendix Table C2 (one persistent decode step): reconstruct, update, readout before
 *     requantization, pack.
 *   - "DAMP: Decay-Aware Mixed-Precision Recurrent-State Quantization", abstract (arXiv v1 and
 *     the later version): high-risk key channels kept in FP16, the remainder in INT8, chosen
 *     offline from quantization-error energy and decay-based persistence.
 *
 * State of one unit (one (slot, head)): D x D, row i = key channel i, column j = value dim j.
 * Logical quantized representation used by the oracle (not the GPU's packed layout):
 *   mask[i]  = 1 -> row i is FP16:  h[i*D + j] holds IEEE binary16 bits
 *   mask[i]  = 0 -> row i is INT8:  c[i*D + j] holds the code, s[i] the fp32 scale
 * Uniform INT8 is the same representation with every mask[i] = 0.
 *
 * Parity status: every function here is pinned by tests under tests/ (closed forms, exact
 * rational brute force, numpy's IEEE float16 and float32 routines). None is "parity unpinned".
 */
#ifndef DAMP_ORACLE_H
#define DAMP_ORACLE_H

#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

/* IEEE 754 binary32 <-> binary16, round to nearest, ties to even; subnormals kept; overflow to
 * +-inf. Array forms convert n values. */
uint16_t oracle_f16_from_f32(float x);
float oracle_f32_from_f16(uint16_t h);
void oracle_f16_from_f32_n(const float* x, uint16_t* h, long n);
void oracle_f32_from_f16_n(const uint16_t* h, float* x, long n);

/* Requantize one row of D binary32 values to symmetric INT8: m = max|x|, s = m/127 (binary32
 * division), c = clamp(round_half_even(x/s), -127, 127) with x/s a binary32 division.
 * s == 0 (m == 0, or m < 127 * 2^-150 so that m/127 rounds to zero) gives all codes 0. */
void oracle_quant_row(int D, const float* x, int8_t* c, float* s);

/* Pack n_units fp32 states S[n][D][D] into the logical representation (mask[n][D]). */
int oracle_quantize(int D, long n_units, const uint8_t* mask, const float* S, uint16_t* h,
                    int8_t* c, float* s, int nthreads);

/* Reconstruct: S[i][j] = c[i][j] * s[i] (INT8 row) or the FP16 value, rounded once to fp32. */
int oracle_dequantize(int D, long n_units, const uint8_t* mask, const uint16_t* h,
                      const int8_t* c, const float* s, float* S, int nthreads);

/* One decode step for n_units independent units.
 *   fmt 0: fp32 state S32[n][D][D] (h, c, s, mask unused, may be NULL)
 *   fmt 1: quantized state (mask, h, c, s); S32 unused
 *   q, k, v: [n][D] binary32 (bf16 inputs arrive already widened, which is exact)
 *   alpha:   [n] (per_key = 0, GDN scalar gate) or [n][D] (per_key = 1, KDA per-key gate)
 *   beta:    [n];  out: [n][D] readout
 * Returns 0, or -1 on an invalid argument. The state is updated in place. */
int oracle_step(int D, long n_units, int fmt, const uint8_t* mask, float* S32, uint16_t* h,
                int8_t* c, float* s, const float* q, const float* k, const float* v,
                const float* alpha, int per_key, const float* beta, float* out, int nthreads);

/* Offline row selection (a harness step, not the decode step):
 *   score[h][i] = mean over slots of (1/D) sum_j S[slot][h][i][j]^2, divided by (1 - abar[h][i])
 * rows[h][0..r) = the r highest scores (ties -> lower index), stored ascending.
 * S is [n_slots][H][D][D]; abar is [H][D]. Returns 0 or -1. */
int oracle_select_rows(int D, int H, long n_slots, const float* S, const double* abar, int r,
                       int32_t* rows, double* score);

/* Budgeted selection with a per-head FP16 row count (offline calibration, not the decode step).
 *   oracle_int8_row_error: sum_j (x_j - s c_j)^2 in binary64 for the INT8 rule's (c, s) of x.
 *   oracle_risk_scores:    score[h][i] = mean over slots of that error for row i of head h,
 *                          divided by (1 - abar[h][i]); S [n_slots][H][D][D], abar [H][D].
 *   oracle_budget_rows:    FP16 rows per slot (all heads) that fit bits_per_value data bits per
 *                          state value, a multiple of g, at most H * r_max; -1 if none fits.
 *   oracle_allocate_rows:  R rows handed out in groups of g by score; r_out [H], map_out [H][D]
 *                          (each head's FP16 rows ascending, then its INT8 rows ascending). */
double oracle_int8_row_error(int D, const float* x);
int oracle_risk_scores(int D, int H, long n_slots, const float* S, const float* abar,
                       double* score);
long oracle_budget_rows(int D, int H, double bits_per_value, int g, int r_max);
int oracle_allocate_rows(int D, int H, const double* score, long R, int g, int r_max,
                         int32_t* r_out, int32_t* map_out);

/* Pre-step: q_hat = q/||q||, k_hat = k/||k|| (zero stays zero), alpha = exp(-softplus(g)),
 * beta = sigmoid(b); binary64, rounded once to binary32. q, k [n][D]; g [n] or [n][D]
 * (per_key); b [n]. Returns 0 or -1. */
int oracle_prestep(int D, long n, const float* q, const float* k, const float* g, int per_key,
                   const float* b, float* q_out, float* k_out, float* alpha_out,
                   float* beta_out);

/* Per-window requantization: within a window of W tokens a unit's state is the exact binary64
 * recurrence started from the reconstruction of (h, c, s), its readouts come from that state,
 * and after the W-th token it is rounded to binary32 and stored with the unit's rule.
 *   Sx double [n][D][D] (the units' exact states, caller-held), t int32 [n] (tokens applied in
 *   the current window; 0 = the window starts with this call's token). Other arguments as in
 *   oracle_step (fmt 1). oracle_window_flush stores every unit with t > 0 and sets t = 0.
 * Return 0 or -1. */
int oracle_window_step(int D, long n_units, const uint8_t* mask, uint16_t* h, int8_t* c,
                       float* s, double* Sx, int32_t* t, int W, const float* q, const float* k,
                       const float* v, const float* alpha, int per_key, const float* beta,
                       float* out, int nthreads);
int oracle_window_flush(int D, long n_units, const uint8_t* mask, uint16_t* h, int8_t* c,
                        float* s, const double* Sx, int32_t* t);

/* STEPQuant-style state: pivot rows in FP16, integer rows with per-row code widths {4, 6, 8},
 * one FP16 row factor per integer row and one FP16 column-scale vector per unit, fitted from X
 * with squared row-impact weights (the fit is written out in oracle.c).
 *   bits [n][D] (16 = pivot, 8, 6, 4), w [n][D] row-impact scores, h [n][D][D] binary16 pivot
 *   values, c [n][D][D] codes, rf [n][D] and cs [n][D] binary16 bits.
 * oracle_stq_step writes the new state to (h2, c2, rf2, cs2), which may alias the inputs, and,
 * when x_out is not NULL, the units' new states X rounded to binary32 [n][D][D].
 * oracle_stq_fit_rows takes the second half of the fit alone: for given column scales cs [n][D]
 * it writes the pivot values, row factors and codes of the states X [n][D][D]. */
int oracle_stq_quantize(int D, long n, const uint8_t* bits, const float* w, const float* S,
                        uint16_t* h, int8_t* c, uint16_t* rf, uint16_t* cs);
int oracle_stq_dequantize(int D, long n, const uint8_t* bits, const uint16_t* h,
                          const int8_t* c, const uint16_t* rf, const uint16_t* cs, float* S);
int oracle_stq_step(int D, long n, const uint8_t* bits, const float* w, const uint16_t* h,
                    const int8_t* c, const uint16_t* rf, const uint16_t* cs, uint16_t* h2,
                    int8_t* c2, uint16_t* rf2, uint16_t* cs2, const float* q, const float* k,
                    const float* v, const float* alpha, int per_key, const float* beta,
                    float* out, float* x_out, int nthreads);
int oracle_stq_fit_rows(int D, long n, const uint8_t* bits, const float* X, const uint16_t* cs,
                        uint16_t* h, int8_t* c, uint16_t* rf);

#ifdef __cplusplus
}
#endif
#endif
