/*
 * oracle.c -- CPU oracle for the GDN / KDA recurrent-state decode step in FP32, uniform INT8
 * and DAMP's FP16 + INT8 layout.
 *
 * TEST INFRASTRUCTURE ONLY (see oracle.h): loaded by the tests, the smoke check and the
 * benchmark's CPU-baseline leg, never by the GPU library or its Python binding.
 *
 * Arithmetic policy. The pages do not fix the precision of the step's intermediate values, so
 * every real-valued quantity of the step (reconstructed state, decayed state, projection,
 * delta, new state, readout) is computed in binary64, in the order the step defines it, with
 * plain loops (no blocking, fusion or reordering). The new state X is rounded once to binary32,
 * the working precision of the recurrent state (the DAMP abstract: states are commonly kept in
 * FP32). Every quantization decision (binary16 rounding, the INT8 scale and the INT8 codes) is
 * taken on that binary32 X, in binary32, which is also the precision the GPU kernels use.
 *
 * Build: gcc -O2 -std=c11 -fopenmp -fPIC -shared -ffp-contract=off -fno-fast-math.
 * -ffp-contract=off keeps every a*b+c as two rounded operations, so the binary32 division
 * and nearbyintf below are exactly the IEEE operations.
 */
#include "oracle.h"

#include <math.h>
#include <stdlib.h>
#include <string.h>

/* ------------------------------------------------------------------------------------------
 * IEEE 754 binary16, written from the format definition (1 sign bit, 5 exponent bits with bias
 * 15, 10 fraction bits; subnormals have spacing 2^-24; the largest finite value is 65504).
 * Round to nearest, ties to even. Binary32 -> binary64 is exact and scaling by a power of two
 * is exact, so the rounding is done on an exact integer multiple count with nearbyint().
 * ---------------------------------------------------------------------------------------- */
static uint16_t f16_from_double(double x) {
  const uint16_t sign = signbit(x) ? 0x8000u : 0u;
  if (isnan(x)) return (uint16_t)(sign | 0x7e00u);
  const double a = fabs(x);
  /* 65520 = 65504 + half of the last binade's spacing (32); at or above it, RNE overflows. */
  if (a >= 65520.0) return (uint16_t)(sign | 0x7c00u);
  if (a == 0.0) return sign;
  int e2;
  (void)frexp(a, &e2); /* a = f * 2^e2 with f in [0.5, 1): a lies in [2^(e2-1), 2^e2) */
  const int E = e2 - 1;
  if (E < -14) {
    /* subnormal range: value = n * 2^-24, n in [0, 1024]; n = 1024 encodes 2^-14 exactly */
    const double n = nearbyint(ldexp(a, 24));
    return (uint16_t)(sign | (uint16_t)n);
  }
  /* normal range: value = n * 2^(E-10), n in [1024, 2048]; n = 2048 carries into E + 1 */
  const double n = nearbyint(ldexp(a, 10 - E));
  const uint32_t bits = ((uint32_t)(E + 15) << 10) + (uint32_t)n - 1024u;
  return (uint16_t)(sign | bits);
}

/* binary32 widens to binary64 exactly, so this is the single rounding of x to binary16 */
uint16_t oracle_f16_from_f32(float xf) { return f16_from_double((double)xf); }

float oracle_f32_from_f16(uint16_t h) {
  const int sign = (h >> 15) & 1;
  const int ex = (h >> 10) & 0x1f;
  const int fr = h & 0x3ff;
  double v;
  if (ex == 0x1f)
    v = fr ? NAN : INFINITY;
  else if (ex == 0)
    v = ldexp((double)fr, -24);
  else
    v = ldexp((double)(1024 + fr), ex - 25);
  return (float)(sign ? -v : v);
}

void oracle_f16_from_f32_n(const float* x, uint16_t* h, long n) {
  for (long i = 0; i < n; ++i) h[i] = oracle_f16_from_f32(x[i]);
}

void oracle_f32_from_f16_n(const uint16_t* h, float* x, long n) {
  for (long i = 0; i < n; ++i) x[i] = oracle_f32_from_f16(h[i]);
}

/* ------------------------------------------------------------------------------------------
 * INT8 row requantization. The pages name only "INT8" for the non-pivot rows (DAMP abstract);
 * the rule used here is symmetric, one fp32 scale per row, scale = row absmax / 127, codes
 * rounded half-to-even and limited to [-127, 127] (code -128 is never produced).
 * ---------------------------------------------------------------------------------------- */
void oracle_quant_row(int D, const float* x, int8_t* c, float* s) {
  float m = 0.0f;
  for (int j = 0; j < D; ++j) {
    const float a = fabsf(x[j]);
    if (a > m) m = a;
  }
  const float sc = m / 127.0f; /* binary32 division, round to nearest even */
  if (sc == 0.0f) {
    /* an all-zero row, or one whose absmax is below 127 * 2^-150 so that m / 127 rounds to
     * zero: scale 0, codes 0 (no code can reconstruct anything else with a zero scale) */
    *s = 0.0f;
    memset(c, 0, (size_t)D);
    return;
  }
  for (int j = 0; j < D; ++j) {
    const float t = x[j] / sc;   /* binary32 division */
    float r = nearbyintf(t);     /* default rounding mode: to nearest, ties to even */
    if (r > 127.0f) r = 127.0f;
    if (r < -127.0f) r = -127.0f;
    c[j] = (int8_t)r;
  }
  *s = sc;
}

/* Reconstructed value of entry (i, j) of a quantized unit, exact in binary64: an 8-bit code
 * times a 24-bit significand fits in 53 bits, and binary16 widens exactly.
 * (Table C2 step 1 of the STEPQuant page: integer codes and scales, or FP16 for pivot units.) */
static double recon(int D, const uint8_t* mask, const uint16_t* h, const int8_t* c,
                    const float* s, int i, int j) {
  if (mask[i]) return (double)oracle_f32_from_f16(h[(long)i * D + j]);
  return (double)c[(long)i * D + j] * (double)s[i];
}

int oracle_quantize(int D, long n_units, const uint8_t* mask, const float* S, uint16_t* h,
                    int8_t* c, float* s, int nthreads) {
  if (D <= 0 || n_units < 0 || !mask || !S || !h || !c || !s) return -1;
  const long DD = (long)D * D;
#pragma omp parallel for schedule(static) num_threads(nthreads > 0 ? nthreads : 1)
  for (long u = 0; u < n_units; ++u) {
    for (int i = 0; i < D; ++i) {
      const float* row = S + u * DD + (long)i * D;
      if (mask[u * D + i]) {
        for (int j = 0; j < D; ++j) h[u * DD + (long)i * D + j] = oracle_f16_from_f32(row[j]);
        memset(c + u * DD + (long)i * D, 0, (size_t)D);
        s[u * D + i] = 0.0f;
      } else {
        for (int j = 0; j < D; ++j) h[u * DD + (long)i * D + j] = 0;
        oracle_quant_row(D, row, c + u * DD + (long)i * D, s + u * D + i);
      }
    }
  }
  return 0;
}

int oracle_dequantize(int D, long n_units, const uint8_t* mask, const uint16_t* h,
                      const int8_t* c, const float* s, float* S, int nthreads) {
  if (D <= 0 || n_units < 0 || !mask || !S || !h || !c || !s) return -1;
  const long DD = (long)D * D;
#pragma omp parallel for schedule(static) num_threads(nthreads > 0 ? nthreads : 1)
  for (long u = 0; u < n_units; ++u)
    for (int i = 0; i < D; ++i)
      for (int j = 0; j < D; ++j)
        S[u * DD + (long)i * D + j] =
            (float)recon(D, mask + u * D, h + u * DD, c + u * DD, s + u * D, i, j);
  return 0;
}

/* ------------------------------------------------------------------------------------------
 * One decode step of one unit, in the order of Table C2 on the STEPQuant page:
 *   1. reconstruct S_hat from codes and scales, or from FP16 for pivot rows (fp32 format: the
 *      stored values);
 *   2. X = D_t S_hat + beta k (v^T - k^T D_t S_hat), with D_t = alpha I (GDN) or diag(alpha)
 *      (KDA; the table's KDA remark and the DAMP abstract's per-key-channel decay);
 *   3. readout y = X^T q, taken from X before requantization;
 *   6. store: FP16 for pivot rows, INT8 codes + scale for the rest (DAMP abstract), or fp32.
 * Steps 4-5 of that table (STEPQuant's dual-axis fitting) are not part of DAMP.
 * work holds D*D + D doubles.
 * ---------------------------------------------------------------------------------------- */
static void step_unit(int D, int fmt, const uint8_t* mask, float* S32, uint16_t* h, int8_t* c,
                      float* s, const float* q, const float* k, const float* v,
                      const float* alpha, int per_key, float beta, float* out, double* work,
                      float* rowbuf) {
  double* X = work;       /* D x D */
  double* u = work + (long)D * D; /* D: k^T D_t S_hat */

  /* steps 1 and 2a: S' = D_t S_hat, held in X */
  for (int i = 0; i < D; ++i) {
    const double a = (double)(per_key ? alpha[i] : alpha[0]);
    for (int j = 0; j < D; ++j) {
      const double sh = fmt == 0 ? (double)S32[(long)i * D + j] : recon(D, mask, h, c, s, i, j);
      X[(long)i * D + j] = a * sh;
    }
  }
  /* step 2b: u_j = sum_i k_i S'_ij, i ascending */
  for (int j = 0; j < D; ++j) {
    double acc = 0.0;
    for (int i = 0; i < D; ++i) acc += (double)k[i] * X[(long)i * D + j];
    u[j] = acc;
  }
  /* step 2c: X_ij = S'_ij + k_i * beta * (v_j - u_j) */
  for (int i = 0; i < D; ++i)
    for (int j = 0; j < D; ++j)
      X[(long)i * D + j] += (double)k[i] * ((double)beta * ((double)v[j] - u[j]));
  /* step 3: y_j = sum_i q_i X_ij from the unquantized X */
  for (int j = 0; j < D; ++j) {
    double acc = 0.0;
    for (int i = 0; i < D; ++i) acc += (double)q[i] * X[(long)i * D + j];
    out[j] = (float)acc;
  }
  /* step 6: round X once to binary32, then store in the unit's format */
  for (int i = 0; i < D; ++i) {
    for (int j = 0; j < D; ++j) rowbuf[j] = (float)X[(long)i * D + j];
    if (fmt == 0) {
      memcpy(S32 + (long)i * D, rowbuf, sizeof(float) * (size_t)D);
    } else if (mask[i]) {
      for (int j = 0; j < D; ++j) h[(long)i * D + j] = oracle_f16_from_f32(rowbuf[j]);
    } else {
      oracle_quant_row(D, rowbuf, c + (long)i * D, s + i);
    }
  }
}

int oracle_step(int D, long n_units, int fmt, const uint8_t* mask, float* S32, uint16_t* h,
                int8_t* c, float* s, const float* q, const float* k, const float* v,
                const float* alpha, int per_key, const float* beta, float* out, int nthreads) {
  if (D <= 0 || n_units < 0 || (fmt != 0 && fmt != 1)) return -1;
  if (!q || !k || !v || !alpha || !beta || !out) return -1;
  if (fmt == 0 && !S32) return -1;
  if (fmt == 1 && (!mask || !h || !c || !s)) return -1;
  const long DD = (long)D * D;
  int bad = 0;
#pragma omp parallel num_threads(nthreads > 0 ? nthreads : 1)
  {
    double* work = (double*)malloc(sizeof(double) * (size_t)(DD + D));
    float* rowbuf = (float*)malloc(sizeof(float) * (size_t)D);
    if (!work || !rowbuf) {
#pragma omp atomic write
      bad = 1;
    }
#pragma omp for schedule(static)
    for (long un = 0; un < n_units; ++un) {
      if (!work || !rowbuf) continue;
      step_unit(D, fmt, fmt ? mask + un * D : NULL, fmt ? NULL : S32 + un * DD,
                fmt ? h + un * DD : NULL, fmt ? c + un * DD : NULL, fmt ? s + un * D : NULL,
                q + un * D, k + un * D, v + un * D, per_key ? alpha + un * D : alpha + un,
                per_key, beta[un], out + un * D, work, rowbuf);
    }
    free(work);
    free(rowbuf);
  }
  return bad ? -1 : 0;
}

/* ------------------------------------------------------------------------------------------
 * Offline selection of high-risk key rows. The DAMP abstract ranks key channels by
 * quantization-error energy together with decay-based error retention and fixes the choice
 * offline. Here error energy is read as the row's mean square (the energy an INT8 row with a
 * row absmax scale spreads its error over) and retention as the geometric-series factor
 * 1/(1 - abar) of a gate that multiplies the state by abar each step.
 * ---------------------------------------------------------------------------------------- */
int oracle_select_rows(int D, int H, long n_slots, const float* S, const double* abar, int r,
                       int32_t* rows, double* score) {
  if (D <= 0 || H <= 0 || n_slots <= 0 || r < 0 || r > D || !S || !abar || !rows || !score)
    return -1;
  const long DD = (long)D * D;
  for (int hh = 0; hh < H; ++hh) {
    for (int i = 0; i < D; ++i) {
      double e = 0.0;
      for (long sl = 0; sl < n_slots; ++sl) {
        const float* row = S + (sl * H + hh) * DD + (long)i * D;
        double ms = 0.0;
        for (int j = 0; j < D; ++j) ms += (double)row[j] * (double)row[j];
        e += ms / (double)D;
      }
      e /= (double)n_slots;
      score[(long)hh * D + i] = e / (1.0 - abar[(long)hh * D + i]);
    }
    /* r rounds of "take the largest remaining score, lower index on ties" */
    char* taken = (char*)calloc((size_t)D, 1);
    if (!taken) return -1;
    for (int t = 0; t < r; ++t) {
      int best = -1;
      for (int i = 0; i < D; ++i) {
        if (taken[i]) continue;
        if (best < 0 || score[(long)hh * D + i] > score[(long)hh * D + best]) best = i;
      }
      taken[best] = 1;
    }
    int n = 0;
    for (int i = 0; i < D; ++i)
      if (taken[i]) rows[(long)hh * r + n++] = i;
    free(taken);
  }
  return 0;
}

/* ------------------------------------------------------------------------------------------
 * Budgeted selection with a per-head FP16 row count. The DAMP abstracts: high-risk key
 * channels are chosen offline from quantization-error energy and decay-based error retention,
 * and kept in FP16 under a fixed total storage budget (9.9 bits per state value on the
 * pages); the remaining rows are INT8. Readings taken here:
 *   - quantization-error energy of a key row = the squared error of storing that row with the
 *     INT8 rule above, sum_j (x_j - s * c_j)^2, averaged over the calibration states;
 *   - retention = 1 / (1 - abar) for a channel whose mean gate is abar (each step multiplies
 *     what the state holds by abar, so an error survives for a geometric series of steps);
 *   - the budget counts data bytes (FP16 rows, INT8 rows, fp32 INT8 scales), and its FP16
 *     rows go to the rows with the largest scores over all heads, handed out in groups of g
 *     rows per head (g = 1 gives a per-row choice), at most r_max per head.
 * ---------------------------------------------------------------------------------------- */

/* Squared INT8 error of one row, in binary64. s * c is exact in binary64 (24-bit significand
 * times a 7-bit integer); the difference x - s*c is exact too (when c != 0 both lie within a
 * factor 256 of s), so only the square and the sum round. */
double oracle_int8_row_error(int D, const float* x) {
  int8_t* c = (int8_t*)malloc((size_t)D);
  if (!c) return -1.0;
  float s = 0.0f;
  oracle_quant_row(D, x, c, &s);
  double e = 0.0;
  for (int j = 0; j < D; ++j) {
    const double d = (double)x[j] - (double)s * (double)c[j];
    e += d * d;
  }
  free(c);
  return e;
}

/* score[h][i] = (sum over slots, ascending, of the row error) / n_slots / (1 - abar[h][i]). */
int oracle_risk_scores(int D, int H, long n_slots, const float* S, const float* abar,
                       double* score) {
  if (D <= 0 || H <= 0 || n_slots <= 0 || !S || !abar || !score) return -1;
  const long DD = (long)D * D;
  for (int hh = 0; hh < H; ++hh) {
    for (int i = 0; i < D; ++i) {
      double e = 0.0;
      for (long sl = 0; sl < n_slots; ++sl)
        e += oracle_int8_row_error(D, S + (sl * H + hh) * DD + (long)i * D);
      e /= (double)n_slots;
      score[(long)hh * D + i] = e / (1.0 - (double)abar[(long)hh * D + i]);
    }
  }
  return 0;
}

/* Data bytes of one head's block with r FP16 rows: 2rD + (D - r)D + 4(D - r). */
static double block_data_bytes(int D, long r) {
  return 2.0 * r * D + (double)(D - r) * D + 4.0 * (D - r);
}

/* The number of FP16 rows, summed over the H heads of a slot, that fits in bits_per_value bits
 * per state value: the largest R, a multiple of g and at most H * r_max, with
 * H * (D^2 + 4D) + (D - 4) * R <= bits_per_value * H * D^2 / 8. -1 if not even R = 0 fits. */
long oracle_budget_rows(int D, int H, double bits_per_value, int g, int r_max) {
  if (D <= 4 || H <= 0 || g <= 0 || r_max < 0 || r_max > D) return -1;
  const double budget = bits_per_value * H * (double)D * D / 8.0;
  long R = -1;
  for (long t = 0; t <= (long)H * r_max; t += g) {
    if ((double)H * block_data_bytes(D, 0) + (double)(D - 4) * t <= budget) R = t;
  }
  return R;
}

/* Allocation of R FP16 rows (R a multiple of g). Per head, the rows are ranked by score, larger
 * first, ties to the lower row index; group j of head h is that ranking's rows j*g .. j*g+g-1
 * and its gain is the sum of their scores, added in ranking order. Groups past r_max / g are
 * never taken. The R / g groups with the largest gains are taken, ties to the lower head and
 * then the lower group index; since a head's gains do not increase along its ranking, each head
 * ends up with a prefix of its ranking, r_h = g * (groups taken). This greedy choice maximises
 * the total score kept in FP16 for the given R (every group costs the same bytes).
 * Outputs r_out[H] and map_out[H][D]: the head's r_h FP16 rows ascending, then its INT8 rows
 * ascending. Returns 0, or -1 on an invalid argument. */
int oracle_allocate_rows(int D, int H, const double* score, long R, int g, int r_max,
                         int32_t* r_out, int32_t* map_out) {
  if (D <= 0 || H <= 0 || g <= 0 || r_max < 0 || r_max > D || R < 0 || R % g != 0 || !score ||
      !r_out || !map_out)
    return -1;
  const int G = r_max / g; /* groups per head that may be taken */
  int32_t* rank = (int32_t*)malloc(sizeof(int32_t) * (size_t)H * D); /* [h][t] -> row */
  double* gain = (double*)malloc(sizeof(double) * (size_t)H * (G > 0 ? G : 1));
  char* taken = (char*)calloc((size_t)H * (G > 0 ? G : 1), 1);
  if (!rank || !gain || !taken) {
    free(rank); free(gain); free(taken);
    return -1;
  }
  for (int hh = 0; hh < H; ++hh) {
    const double* sc = score + (long)hh * D;
    /* selection sort by (score desc, index asc) */
    char* used = (char*)calloc((size_t)D, 1);
    for (int t = 0; t < D; ++t) {
      int best = -1;
      for (int i = 0; i < D; ++i) {
        if (used[i]) continue;
        if (best < 0 || sc[i] > sc[best]) best = i;
      }
      used[best] = 1;
      rank[(long)hh * D + t] = best;
    }
    free(used);
    for (int j = 0; j < G; ++j) {
      double gsum = 0.0;
      for (int t = j * g; t < j * g + g; ++t) gsum += sc[rank[(long)hh * D + t]];
      gain[(long)hh * G + j] = gsum;
    }
  }
  long want = R / g;
  if (want > (long)H * G) want = (long)H * G;
  for (long t = 0; t < want; ++t) {
    long best = -1;
    for (long x = 0; x < (long)H * G; ++x) {
      if (taken[x]) continue;
      if (best < 0 || gain[x] > gain[best]) best = x; /* x ascends in (head, group) order */
    }
    taken[best] = 1;
  }
  for (int hh = 0; hh < H; ++hh) {
    int r = 0;
    for (int j = 0; j < G; ++j) r += taken[(long)hh * G + j] ? g : 0;
    r_out[hh] = r;
    char* fp16 = (char*)calloc((size_t)D, 1);
    for (int t = 0; t < r; ++t) fp16[rank[(long)hh * D + t]] = 1;
    int n = 0;
    for (int i = 0; i < D; ++i)
      if (fp16[i]) map_out[(long)hh * D + n++] = i;
    for (int i = 0; i < D; ++i)
      if (!fp16[i]) map_out[(long)hh * D + n++] = i;
    free(fp16);
  }
  free(rank); free(gain); free(taken);
  return 0;
}

/* ------------------------------------------------------------------------------------------
 * Pre-step (the inputs of the decode step as a GDN / KDA layer produces them). The step's q and
 * k are unit vectors and its gates come from logits: q_hat = q / ||q||_2, k_hat = k / ||k||_2,
 * alpha = exp(-softplus(g)) = 1 / (1 + e^g), beta = 1 / (1 + e^-b). A zero vector stays zero
 * (no division by zero). Each value is computed in binary64 and rounded once to binary32, the
 * precision the step takes its inputs in.
 *   q, k [n][D]; g [n] (per_key = 0) or [n][D] (per_key = 1); b [n]; outputs of the same shapes.
 * ---------------------------------------------------------------------------------------- */
static double logistic(double x) { return 1.0 / (1.0 + exp(-x)); }

int oracle_prestep(int D, long n, const float* q, const float* k, const float* g, int per_key,
                   const float* b, float* q_out, float* k_out, float* alpha_out,
                   float* beta_out) {
  if (D <= 0 || n < 0 || !q || !k || !g || !b || !q_out || !k_out || !alpha_out || !beta_out)
    return -1;
  for (long u = 0; u < n; ++u) {
    const float* vin[2] = {q + u * D, k + u * D};
    float* vout[2] = {q_out + u * D, k_out + u * D};
    for (int t = 0; t < 2; ++t) {
      double ss = 0.0;
      for (int i = 0; i < D; ++i) ss += (double)vin[t][i] * (double)vin[t][i];
      const double nrm = sqrt(ss);
      for (int i = 0; i < D; ++i) vout[t][i] = nrm > 0.0 ? (float)((double)vin[t][i] / nrm) : 0.0f;
    }
    const long ng = per_key ? D : 1;
    for (long i = 0; i < ng; ++i) alpha_out[u * ng + i] = (float)logistic(-(double)g[u * ng + i]);
    beta_out[u] = (float)logistic((double)b[u]);
  }
  return 0;
}

/* ------------------------------------------------------------------------------------------
 * Per-window requantization (the LeapQuant page, abstract: the low-bit state stays fixed for a
 * window of tokens, the window's updates are held in high precision, outputs come from the
 * fixed state together with those updates, and the state is quantized once, at the window's
 * end). Read here as: within a window a unit's state is the exact (binary64) recurrence started
 * from the reconstruction of its low-bit state, each readout is taken from that state, and after
 * the window's W-th token the state is rounded once to binary32 and stored with the unit's rule
 * (FP16 rows RNE, INT8 rows absmax / 127). W = 1 is the per-token step.
 *   Sx  binary64 [n][D][D]: each unit's state within its window (held by the caller)
 *   t   [n]: tokens of the current window already applied (0: the window starts with this one)
 * ---------------------------------------------------------------------------------------- */
static void store_unit(int D, const uint8_t* mask, uint16_t* h, int8_t* c, float* s,
                       const double* Sx, float* rowbuf) {
  for (int i = 0; i < D; ++i) {
    for (int j = 0; j < D; ++j) rowbuf[j] = (float)Sx[(long)i * D + j];
    if (mask[i]) {
      for (int j = 0; j < D; ++j) h[(long)i * D + j] = oracle_f16_from_f32(rowbuf[j]);
      memset(c + (long)i * D, 0, (size_t)D);
      s[i] = 0.0f;
    } else {
      for (int j = 0; j < D; ++j) h[(long)i * D + j] = 0;
      oracle_quant_row(D, rowbuf, c + (long)i * D, s + i);
    }
  }
}

int oracle_window_step(int D, long n_units, const uint8_t* mask, uint16_t* h, int8_t* c,
                       float* s, double* Sx, int32_t* t, int W, const float* q, const float* k,
                       const float* v, const float* alpha, int per_key, const float* beta,
                       float* out, int nthreads) {
  if (D <= 0 || n_units < 0 || W < 1 || !mask || !h || !c || !s || !Sx || !t || !q || !k ||
      !v || !alpha || !beta || !out)
    return -1;
  const long DD = (long)D * D;
  int bad = 0;
#pragma omp parallel num_threads(nthreads > 0 ? nthreads : 1)
  {
    double* u = (double*)malloc(sizeof(double) * (size_t)D);
    float* rowbuf = (float*)malloc(sizeof(float) * (size_t)D);
    if (!u || !rowbuf) {
#pragma omp atomic write
      bad = 1;
    }
#pragma omp for schedule(static)
    for (long un = 0; un < n_units; ++un) {
      if (!u || !rowbuf) continue;
      const uint8_t* mk = mask + un * D;
      double* X = Sx + un * DD;
      if (t[un] < 0 || t[un] >= W) continue;
      if (t[un] == 0) /* a window starts: the exact state is the reconstruction */
        for (int i = 0; i < D; ++i)
          for (int j = 0; j < D; ++j)
            X[(long)i * D + j] = recon(D, mk, h + un * DD, c + un * DD, s + un * D, i, j);
      const float* qu = q + un * D;
      const float* ku = k + un * D;
      const float* vu = v + un * D;
      const float* au = per_key ? alpha + un * D : alpha + un;
      /* the decode step on the exact state: S' = D_t S, u = S'^T k, X = S' + k beta (v - u) */
      for (int i = 0; i < D; ++i) {
        const double a = (double)(per_key ? au[i] : au[0]);
        for (int j = 0; j < D; ++j) X[(long)i * D + j] *= a;
      }
      for (int j = 0; j < D; ++j) {
        double acc = 0.0;
        for (int i = 0; i < D; ++i) acc += (double)ku[i] * X[(long)i * D + j];
        u[j] = acc;
      }
      for (int i = 0; i < D; ++i)
        for (int j = 0; j < D; ++j)
          X[(long)i * D + j] += (double)ku[i] * ((double)beta[un] * ((double)vu[j] - u[j]));
      for (int j = 0; j < D; ++j) {
        double acc = 0.0;
        for (int i = 0; i < D; ++i) acc += (double)qu[i] * X[(long)i * D + j];
        out[un * D + j] = (float)acc;
      }
      t[un] += 1;
      if (t[un] == W) {
        store_unit(D, mk, h + un * DD, c + un * DD, s + un * D, X, rowbuf);
        t[un] = 0;
      }
    }
    free(u);
    free(rowbuf);
  }
  for (long un = 0; un < n_units; ++un)
    if (t[un] < 0 || t[un] >= W) bad = 1;
  return bad ? -1 : 0;
}

/* Store every unit with pending tokens (t > 0) from its exact state and start a new window. */
int oracle_window_flush(int D, long n_units, const uint8_t* mask, uint16_t* h, int8_t* c,
                        float* s, const double* Sx, int32_t* t) {
  if (D <= 0 || n_units < 0 || !mask || !h || !c || !s || !Sx || !t) return -1;
  const long DD = (long)D * D;
  float* rowbuf = (float*)malloc(sizeof(float) * (size_t)D);
  if (!rowbuf) return -1;
  for (long un = 0; un < n_units; ++un) {
    if (t[un] > 0) store_unit(D, mask + un * D, h + un * DD, c + un * DD, s + un * D, Sx + un * DD, rowbuf);
    t[un] = 0;
  }
  free(rowbuf);
  return 0;
}

/* ------------------------------------------------------------------------------------------
 * STEPQuant-style state (the STEPQuant page: Table C2 steps 1-6, Table C1 for KDA, Table D3).
 * Each key row of a head is a pivot (kept in FP16) or an integer row with its own code width
 * b in {4, 6, 8} (a frozen precision map); the integer rows share one column-scale vector per
 * head and carry one row factor each, both stored in FP16; entry (i, j) of an integer row is
 * code_ij * rf_i * cs_j. The page names the fit (a dual-axis fit aware of key rows; for KDA a
 * single column-scale vector per head, fitted over the integer rows with each row weighted by
 * the square of its row-impact score) but not its formulas; the reading taken here, for the
 * non-pivot rows N of a unit:
 *   cs_j = fp16( sqrt( sum_{i in N} w_i^2 X_ij^2 / sum_{i in N} w_i^2 ) )   (binary64, then
 *          binary16 RNE; all w_i = 0 is read as all w_i = 1)
 *   rf_i = fp16( fl32( max_{j: cs_j > 0} fl32(|X_ij| / cs_j) / qmax_i ) ),  qmax = 2^(b-1) - 1
 *   code = clamp(rint(fl32(X_ij / fl32(rf_i cs_j))), -qmax, qmax) when rf_i cs_j > 0, else 0
 * with w_i the row-impact score (an input, as on the page). rf_i cs_j is exact in binary32 (two
 * 11-bit significands), so the decisions are taken in binary32 on that product.
 * Logical arrays per unit: bits [D] (16 = pivot, or 8, 6, 4), w [D], h [D][D] (binary16 bits of
 * the pivot rows, 0 elsewhere), c [D][D] (codes, 0 on pivot rows), rf [D] (binary16 bits, 0 on
 * pivot rows), cs [D] (binary16 bits).
 * ---------------------------------------------------------------------------------------- */
static int stq_qmax(int b) { return (1 << (b - 1)) - 1; }

/* The fit's first half: the column scales of one unit from its binary32 state X. */
static void stq_fit_columns(int D, const uint8_t* bits, const float* w, const float* X,
                            uint16_t* cs) {
  double sw = 0.0;
  for (int i = 0; i < D; ++i)
    if (bits[i] != 16) sw += (double)w[i] * (double)w[i];
  const int unweighted = !(sw > 0.0);
  if (unweighted) {
    sw = 0.0;
    for (int i = 0; i < D; ++i)
      if (bits[i] != 16) sw += 1.0;
  }
  for (int j = 0; j < D; ++j) {
    double acc = 0.0;
    for (int i = 0; i < D; ++i) {
      if (bits[i] == 16) continue;
      const double wi = unweighted ? 1.0 : (double)w[i];
      acc += wi * wi * (double)X[(long)i * D + j] * (double)X[(long)i * D + j];
    }
    cs[j] = sw > 0.0 ? f16_from_double(sqrt(acc / sw)) : 0; /* one rounding to binary16 */
  }
}

/* The fit's second half, given the column scales: pivot values, row factors and codes. */
static void stq_fit_rows(int D, const uint8_t* bits, const float* X, const uint16_t* cs,
                         uint16_t* h, int8_t* c, uint16_t* rf) {
  for (int i = 0; i < D; ++i) {
    const float* x = X + (long)i * D;
    if (bits[i] == 16) {
      for (int j = 0; j < D; ++j) {
        h[(long)i * D + j] = oracle_f16_from_f32(x[j]);
        c[(long)i * D + j] = 0;
      }
      rf[i] = 0;
      continue;
    }
    const int qm = stq_qmax(bits[i]);
    float m = 0.0f;
    for (int j = 0; j < D; ++j) {
      const float csj = oracle_f32_from_f16(cs[j]);
      if (csj > 0.0f) {
        const float a = fabsf(x[j]) / csj;
        if (a > m) m = a;
      }
    }
    rf[i] = oracle_f16_from_f32(m / (float)qm);
    const float rfi = oracle_f32_from_f16(rf[i]);
    for (int j = 0; j < D; ++j) {
      h[(long)i * D + j] = 0;
      const float sc = rfi * oracle_f32_from_f16(cs[j]); /* exact */
      float code = 0.0f;
      if (sc > 0.0f) {
        code = nearbyintf(x[j] / sc);
        if (code > (float)qm) code = (float)qm;
        if (code < (float)-qm) code = (float)-qm;
      }
      c[(long)i * D + j] = (int8_t)code;
    }
  }
}

static void stq_store_unit(int D, const uint8_t* bits, const float* w, const float* X,
                           uint16_t* h, int8_t* c, uint16_t* rf, uint16_t* cs) {
  stq_fit_columns(D, bits, w, X, cs);
  stq_fit_rows(D, bits, X, cs, h, c, rf);
}

static double stq_recon(int D, const uint8_t* bits, const uint16_t* h, const int8_t* c,
                        const uint16_t* rf, const uint16_t* cs, int i, int j) {
  if (bits[i] == 16) return (double)oracle_f32_from_f16(h[(long)i * D + j]);
  return (double)c[(long)i * D + j] * (double)oracle_f32_from_f16(rf[i]) *
         (double)oracle_f32_from_f16(cs[j]);
}

static int stq_bits_ok(int D, const uint8_t* bits) {
  for (int i = 0; i < D; ++i)
    if (bits[i] != 16 && bits[i] != 8 && bits[i] != 6 && bits[i] != 4) return 0;
  return 1;
}

int oracle_stq_quantize(int D, long n, const uint8_t* bits, const float* w, const float* S,
                        uint16_t* h, int8_t* c, uint16_t* rf, uint16_t* cs) {
  if (D <= 0 || n < 0 || !bits || !w || !S || !h || !c || !rf || !cs) return -1;
  const long DD = (long)D * D;
  for (long u = 0; u < n; ++u) {
    if (!stq_bits_ok(D, bits + u * D)) return -1;
    stq_store_unit(D, bits + u * D, w + u * D, S + u * DD, h + u * DD, c + u * DD, rf + u * D,
                   cs + u * D);
  }
  return 0;
}

int oracle_stq_dequantize(int D, long n, const uint8_t* bits, const uint16_t* h,
                          const int8_t* c, const uint16_t* rf, const uint16_t* cs, float* S) {
  if (D <= 0 || n < 0 || !bits || !h || !c || !rf || !cs || !S) return -1;
  const long DD = (long)D * D;
  for (long u = 0; u < n; ++u)
    for (int i = 0; i < D; ++i)
      for (int j = 0; j < D; ++j)
        S[u * DD + (long)i * D + j] = (float)stq_recon(D, bits + u * D, h + u * DD, c + u * DD,
                                                       rf + u * D, cs + u * D, i, j);
  return 0;
}

/* One decode step on STEPQuant-style states: Table C2 steps 1-3 as in oracle_step (binary64,
 * X rounded once to binary32), then steps 4-6 with the fit above. The new state goes to
 * (h2, c2, rf2, cs2), which may be the input arrays (in place) or others (the old
 * representation kept for its readers, Table C2 step 6). */
int oracle_stq_step(int D, long n, const uint8_t* bits, const float* w, const uint16_t* h,
                    const int8_t* c, const uint16_t* rf, const uint16_t* cs, uint16_t* h2,
                    int8_t* c2, uint16_t* rf2, uint16_t* cs2, const float* q, const float* k,
                    const float* v, const float* alpha, int per_key, const float* beta,
                    float* out, float* x_out, int nthreads) {
  if (D <= 0 || n < 0 || !bits || !w || !h || !c || !rf || !cs || !h2 || !c2 || !rf2 || !cs2 ||
      !q || !k || !v || !alpha || !beta || !out)
    return -1;
  const long DD = (long)D * D;
  for (long u = 0; u < n; ++u)
    if (!stq_bits_ok(D, bits + u * D)) return -1;
  int bad = 0;
#pragma omp parallel num_threads(nthreads > 0 ? nthreads : 1)
  {
    double* X = (double*)malloc(sizeof(double) * (size_t)(DD + D));
    float* Xf = (float*)malloc(sizeof(float) * (size_t)DD);
    if (!X || !Xf) {
#pragma omp atomic write
      bad = 1;
    }
#pragma omp for schedule(static)
    for (long un = 0; un < n; ++un) {
      if (!X || !Xf) continue;
      double* uu = X + DD;
      const uint8_t* bt = bits + un * D;
      const float* ku = k + un * D;
      const float* qu = q + un * D;
      const float* vu = v + un * D;
      const float* au = per_key ? alpha + un * D : alpha + un;
      for (int i = 0; i < D; ++i) {
        const double a = (double)(per_key ? au[i] : au[0]);
        for (int j = 0; j < D; ++j)
          X[(long)i * D + j] = a * stq_recon(D, bt, h + un * DD, c + un * DD, rf + un * D,
                                             cs + un * D, i, j);
      }
      for (int j = 0; j < D; ++j) {
        double acc = 0.0;
        for (int i = 0; i < D; ++i) acc += (double)ku[i] * X[(long)i * D + j];
        uu[j] = acc;
      }
      for (int i = 0; i < D; ++i)
        for (int j = 0; j < D; ++j)
          X[(long)i * D + j] += (double)ku[i] * ((double)beta[un] * ((double)vu[j] - uu[j]));
      for (int j = 0; j < D; ++j) {
        double acc = 0.0;
        for (int i = 0; i < D; ++i) acc += (double)qu[i] * X[(long)i * D + j];
        out[un * D + j] = (float)acc;
      }
      for (long e = 0; e < DD; ++e) Xf[e] = (float)X[e];
      if (x_out) memcpy(x_out + un * DD, Xf, sizeof(float) * (size_t)DD);
      stq_store_unit(D, bt, w + un * D, Xf, h2 + un * DD, c2 + un * DD, rf2 + un * D, cs2 + un * D);
    }
    free(X);
    free(Xf);
  }
  return bad ? -1 : 0;
}

/* The second half of the fit for given column scales cs [n][D] (binary16 bits): pivot values,
 * row factors and codes of n units from their binary32 states X [n][D][D]. */
int oracle_stq_fit_rows(int D, long n, const uint8_t* bits, const float* X, const uint16_t* cs,
                        uint16_t* h, int8_t* c, uint16_t* rf) {
  if (D <= 0 || n < 0 || !bits || !X || !cs || !h || !c || !rf) return -1;
  const long DD = (long)D * D;
  for (long u = 0; u < n; ++u) {
    if (!stq_bits_ok(D, bits + u * D)) return -1;
    stq_fit_rows(D, bits + u * D, X + u * DD, cs + u * D, h + u * DD, c + u * DD, rf + u * D);
  }
  return 0;
}
