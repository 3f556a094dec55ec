/*
 * nvfp4_oracle.c -- plain, slow CPU oracle for the NVFP4 weight-only GEMM.
 *
 * TEST INFRASTRUCTURE ONLY.  Nothing in the product path may include, link,
 * load or call this file.  It shares no code, header, table or constant
 * generator with the HIP library; it exists so that the tests and the
 * benchmark's CPU baseline have an independent statement of what the method
 * computes.
 *
 * Sources (page titles; the pages state only the format's shape, the rest is
 * the format definition written out in the last item):
 *  - "The Blackwell Architectural Split: NVFP4, Attention, and Consumer
 *    Silicon", section "Preserving precision -- dual-tier scale handling":
 *    an NVFP4 value has 1 sign bit, 2 exponent bits and 1 mantissa bit, and
 *    the format combines a per-tensor global scale with one block scale for
 *    every 16 values.
 *  - same page, section "The Breakthrough The A4Q Kernel": dequantization
 *    works on 16 low-bit values at a time (one block).
 *  - "The SM120 FP4 GEMM Kernel Investigation", section "The Context":
 *    the deployed model keeps 4-bit floating-point weights and BF16
 *    activations (the W4A16 operating point).
 *  - "The FP4 Frontier", Finding 6: about 4.5 stored bits per weight
 *    (4 bits of value plus an 8-bit scale shared by 16 weights).
 *  - The format definition implemented here fixes the rest: the E2M1 value set
 *    {0, 0.5, 1, 1.5, 2, 3, 4, 6} with a sign, an FP8-E4M3 block scale equal
 *    to the block amax / 6 rounded to E4M3, a global scale equal to the
 *    tensor amax / (6 * 448), and an FP32-accumulate GEMM.
 *
 * Readings taken where the sources are silent:
 *  R1 E2M1 exponent bias is 1 -- the only bias that reproduces the value set.
 *  R2 E4M3 is the OCP "FN" variant (max 448, no infinities, 0x7F/0xFF NaN);
 *     448 as the largest finite value identifies it.
 *  R3 The global scale g = fl32(amax / 2688) is the decode-direction factor;
 *     block scales are stored relative to it, s = E4M3(fl32(fl32(amax_b/6)/g)),
 *     which is the only reading under which every tensor fits E4M3's range.
 *  R4 "Rounded" means round-to-nearest, ties to the even code, saturating at
 *     the largest finite value (448 for E4M3, 6 for E2M1).
 *  R5 Element code: q = fl32(|w| / fl32(s_dec * g)), magnitude = E2M1 RNE of
 *     q, sign bit copied from w (so -0 and small negatives give code 0x8).
 *     If s_dec * g == 0 the magnitude is 0.  An all-zero tensor has g = 0.
 *  R6 Packing: byte j of a row holds element 2j in the low nibble and
 *     element 2j+1 in the high nibble; scales are row-major [rows][k/16].
 *  R7 Non-finite weights make quantize report an error; outputs unspecified.
 *  R8 The reference product is accumulated in double; each product
 *     x * w_dec is exact in double.
 *
 * Build: gcc -O2 -fopenmp -ffp-contract=off -fno-fast-math -shared -fPIC.
 * All single-precision steps are written as separate float operations so the
 * compiler evaluates each one in IEEE binary32 with round-to-nearest-even.
 */
#include <stdint.h>
#include <stddef.h>
#include <string.h>
#include <math.h>

#define ORC_OK 0
#define ORC_ERR_ARG 1
#define ORC_ERR_NONFINITE 2

/* ---- scalar helpers ---------------------------------------------------- */

static float bf16_to_float(uint16_t h) {
  uint32_t u = (uint32_t)h << 16;
  float f;
  memcpy(&f, &u, sizeof f);
  return f;
}

/* E2M1 decode (R1): s = bit 3, e = bits 2..1, m = bit 0.
 * e == 0: (-1)^s * m * 0.5 ; e >= 1: (-1)^s * 2^(e-1) * (1 + m/2). */
double orc_e2m1_value(unsigned code) {
  unsigned s = (code >> 3) & 1u, e = (code >> 1) & 3u, m = code & 1u;
  double mag = (e == 0) ? 0.5 * (double)m : ldexp(1.0 + 0.5 * (double)m, (int)e - 1);
  return s ? -mag : mag;
}

/* E4M3 (OCP FN) decode (R2): s = bit 7, e = bits 6..3 (bias 7), m = bits 2..0.
 * e == 0: (-1)^s * m/8 * 2^-6 ; e == 15 and m == 7: NaN ; else
 * (-1)^s * (1 + m/8) * 2^(e-7). */
double orc_e4m3_value(unsigned code) {
  unsigned s = (code >> 7) & 1u, e = (code >> 3) & 15u, m = code & 7u;
  double mag;
  if (e == 15u && m == 7u) return NAN;
  if (e == 0u) mag = ldexp((double)m / 8.0, -6);
  else mag = ldexp(1.0 + (double)m / 8.0, (int)e - 7);
  return s ? -mag : mag;
}

/* Round a non-negative float to the nearest member of an ascending table of
 * non-negative values (codes 0..count-1, code i has value tab[i]), ties to the
 * even code, saturating at the last entry (R4).  Midpoints of neighbouring
 * table values have at most one more significant bit than the values, so the
 * comparison against the midpoint is exact in double. */
static unsigned round_to_table(double x, const double* tab, unsigned count) {
  unsigned lo = 0, hi = count - 1u;  /* largest i with tab[i] <= x */
  if (x >= tab[count - 1u]) return count - 1u;
  while (lo < hi) {
    unsigned mid = (lo + hi + 1u) / 2u;
    if (tab[mid] <= x) lo = mid; else hi = mid - 1u;
  }
  {
    double midpoint = 0.5 * (tab[lo] + tab[lo + 1u]);
    if (x > midpoint) return lo + 1u;
    if (x < midpoint) return lo;
    return (lo & 1u) ? lo + 1u : lo;  /* tie: the even code */
  }
}

static double e4m3_table[127];  /* codes 0x00..0x7E, ascending */
static double e2m1_table[8];     /* codes 0..7 */
static int tables_ready = 0;

static void make_tables(void) {
  unsigned c;
  if (tables_ready) return;
  for (c = 0; c < 127u; ++c) e4m3_table[c] = orc_e4m3_value(c);
  for (c = 0; c < 8u; ++c) e2m1_table[c] = orc_e2m1_value(c);
  tables_ready = 1;
}

/* E4M3 encode of a non-negative finite float (R4): nearest, ties-to-even,
 * saturating at 448 (code 0x7E).  The sign bit of the result is always 0. */
uint8_t orc_e4m3_encode(float x) {
  make_tables();
  return (uint8_t)round_to_table((double)x, e4m3_table, 127u);
}

/* E2M1 magnitude encode of a non-negative float (R4): 3-bit code, nearest,
 * ties-to-even, saturating at 6.0 (code 7).  +inf saturates as well. */
uint8_t orc_e2m1_encode_mag(float q) {
  make_tables();
  return (uint8_t)round_to_table((double)q, e2m1_table, 8u);
}

void orc_e4m3_encode_array(const float* x, int64_t n, uint8_t* out) {
  int64_t i;
  make_tables();
#pragma omp parallel for schedule(static)
  for (i = 0; i < n; ++i) out[i] = orc_e4m3_encode(x[i]);
}

void orc_e2m1_encode_mag_array(const float* q, int64_t n, uint8_t* out) {
  int64_t i;
  make_tables();
#pragma omp parallel for schedule(static)
  for (i = 0; i < n; ++i) out[i] = orc_e2m1_encode_mag(q[i]);
}

/* ---- quantize ---------------------------------------------------------- */

/* Global scale (R3): g = fl32(amax / 2688), 2688 = 6 * 448. */
float orc_global_scale(float amax) {
  float denom = 2688.0f;
  return amax / denom;
}

/* Block scale code (R3, R4) from the block amax and the global scale. */
uint8_t orc_block_scale_code(float amax_b, float g) {
  float six = 6.0f, t, s;
  if (g == 0.0f) return 0u;
  t = amax_b / six;
  s = t / g;
  return orc_e4m3_encode(s);
}

/* Element code (R5) from the element, its decoded block scale and g. */
uint8_t orc_element_code(float w, float s_dec, float g) {
  float d = s_dec * g;
  uint8_t mag;
  unsigned sign = signbit(w) ? 1u : 0u;
  if (d == 0.0f) {
    mag = 0u;
  } else {
    float q = fabsf(w) / d;
    mag = orc_e2m1_encode_mag(q);
  }
  return (uint8_t)((sign << 3) | mag);
}

/* Quantize `batch` row-major BF16 tensors of shape [n][k] (k % 16 == 0).
 * Outputs: packed [batch][n][k/2] (R6), scales [batch][n][k/16], g [batch].
 * Returns ORC_ERR_NONFINITE if any tensor holds a NaN or infinity (R7). */
int orc_quantize(const uint16_t* w, int64_t batch, int64_t n, int64_t k,
                 uint8_t* packed, uint8_t* scales, float* g_out) {
  int64_t t;
  int status = ORC_OK;
  if (batch < 0 || n < 0 || k < 0 || (k % 16) != 0) return ORC_ERR_ARG;
  make_tables();
  for (t = 0; t < batch; ++t) {
    const uint16_t* wt = w + t * n * k;
    uint8_t* pt = packed + t * n * (k / 2);
    uint8_t* st = scales + t * n * (k / 16);
    int64_t i, r;
    float amax = 0.0f, g;
    int nonfinite = 0;
    /* pass 1: tensor amax (exact: max of magnitudes) */
    for (i = 0; i < n * k; ++i) {
      float v = bf16_to_float(wt[i]);
      if (!isfinite(v)) { nonfinite = 1; break; }
      if (fabsf(v) > amax) amax = fabsf(v);
    }
    if (nonfinite) { status = ORC_ERR_NONFINITE; continue; }
    g = orc_global_scale(amax);
    g_out[t] = g;
    /* pass 2: per 16-block scale, element codes, packing */
#pragma omp parallel for schedule(static)
    for (r = 0; r < n; ++r) {
      int64_t b;
      for (b = 0; b < k / 16; ++b) {
        const uint16_t* blk = wt + r * k + b * 16;
        float amax_b = 0.0f, s_dec;
        uint8_t code[16], sc;
        int j;
        for (j = 0; j < 16; ++j) {
          float v = fabsf(bf16_to_float(blk[j]));
          if (v > amax_b) amax_b = v;
        }
        sc = orc_block_scale_code(amax_b, g);
        st[r * (k / 16) + b] = sc;
        s_dec = (float)orc_e4m3_value(sc);  /* exact in float */
        for (j = 0; j < 16; ++j) code[j] = orc_element_code(bf16_to_float(blk[j]), s_dec, g);
        for (j = 0; j < 8; ++j)
          pt[r * (k / 2) + b * 8 + j] = (uint8_t)(code[2 * j] | (code[2 * j + 1] << 4));
      }
    }
  }
  return status;
}

/* Decoded weight without the global scale: w_dec[r][c] = e2m1 * s_dec, one
 * tensor [n][k] (exact in double; also exact in bf16, checked by the tests). */
void orc_dequant(const uint8_t* packed, const uint8_t* scales, int64_t n, int64_t k,
                 double* w_dec) {
  int64_t r;
#pragma omp parallel for schedule(static)
  for (r = 0; r < n; ++r) {
    int64_t c;
    for (c = 0; c < k; ++c) {
      uint8_t byte = packed[r * (k / 2) + c / 2];
      unsigned code = (c % 2 == 0) ? (byte & 15u) : (byte >> 4);
      double s = orc_e4m3_value(scales[r * (k / 16) + c / 16]);
      w_dec[r * k + c] = orc_e2m1_value(code) * s;
    }
  }
}

/* ---- GEMM -------------------------------------------------------------- */

/* One output element: y = g * sum_k x[k] * w_dec[k] (R8) and the error scale
 * D = |g| * sum_k |x[k] * w_dec[k]|, both in double. */
static void dot_row(const uint16_t* xrow, const uint8_t* prow, const uint8_t* srow,
                    int64_t k, float g, double* y, double* d) {
  double acc = 0.0, mag = 0.0;
  int64_t c;
  for (c = 0; c < k; ++c) {
    uint8_t byte = prow[c / 2];
    unsigned code = (c % 2 == 0) ? (byte & 15u) : (byte >> 4);
    double wv = orc_e2m1_value(code) * orc_e4m3_value(srow[c / 16]);
    double p = (double)bf16_to_float(xrow[c]) * wv;
    acc += p;
    mag += fabs(p);
  }
  *y = (double)g * acc;
  *d = fabs((double)g) * mag;
}

/* Dense: x [m][k] bf16, weight (packed [n][k/2], scales [n][k/16], g);
 * y, d: [m][n] double. */
int orc_gemm(const uint16_t* x, int64_t m, int64_t n, int64_t k,
             const uint8_t* packed, const uint8_t* scales, float g,
             double* y, double* d) {
  int64_t i;
  if (m < 0 || n < 0 || k < 0 || (k % 16) != 0) return ORC_ERR_ARG;
#pragma omp parallel for schedule(dynamic, 1)
  for (i = 0; i < m; ++i) {
    int64_t j;
    for (j = 0; j < n; ++j)
      dot_row(x + i * k, packed + j * (k / 2), scales + j * (k / 16), k, g,
              &y[i * n + j], &d[i * n + j]);
  }
  return ORC_OK;
}

/* Dense, only at `count` sampled (row, col) positions. */
int orc_gemm_sampled(const uint16_t* x, int64_t m, int64_t n, int64_t k,
                     const uint8_t* packed, const uint8_t* scales, float g,
                     const int64_t* rows, const int64_t* cols, int64_t count,
                     double* y, double* d) {
  int64_t t;
  if (m < 0 || n < 0 || k < 0 || (k % 16) != 0) return ORC_ERR_ARG;
  for (t = 0; t < count; ++t)
    if (rows[t] < 0 || rows[t] >= m || cols[t] < 0 || cols[t] >= n) return ORC_ERR_ARG;
#pragma omp parallel for schedule(dynamic, 16)
  for (t = 0; t < count; ++t)
    dot_row(x + rows[t] * k, packed + cols[t] * (k / 2), scales + cols[t] * (k / 16), k, g,
            &y[t], &d[t]);
  return ORC_OK;
}

/* Offsets are valid when offsets[0] == 0, offsets[E] == rows and they never
 * decrease. */
static int offsets_valid(const int32_t* offsets, int64_t rows, int64_t E) {
  int64_t e;
  if (E < 0 || offsets[0] != 0 || (int64_t)offsets[E] != rows) return 0;
  for (e = 0; e < E; ++e)
    if (offsets[e + 1] < offsets[e]) return 0;
  return 1;
}

/* Grouped: rows [offsets[e], offsets[e+1]) of x use expert e's weight
 * (packed [E][n][k/2], scales [E][n][k/16], g [E]); y, d: [rows][n]. */
int orc_grouped_gemm(const uint16_t* x, int64_t rows, const int32_t* offsets, int64_t E,
                     int64_t n, int64_t k, const uint8_t* packed, const uint8_t* scales,
                     const float* g, double* y, double* d) {
  int64_t e;
  if (rows < 0 || n < 0 || k < 0 || (k % 16) != 0) return ORC_ERR_ARG;
  if (!offsets_valid(offsets, rows, E)) return ORC_ERR_ARG;
  for (e = 0; e < E; ++e) {
    int64_t r0 = offsets[e], cnt = (int64_t)offsets[e + 1] - offsets[e];
    if (cnt == 0) continue;
    orc_gemm(x + r0 * k, cnt, n, k, packed + e * n * (k / 2), scales + e * n * (k / 16),
             g[e], y + r0 * n, d + r0 * n);
  }
  return ORC_OK;
}

/* Grouped, only at sampled (row, col) positions; the expert of a row is the
 * segment that holds it. */
int orc_grouped_gemm_sampled(const uint16_t* x, int64_t rows, const int32_t* offsets,
                             int64_t E, int64_t n, int64_t k, const uint8_t* packed,
                             const uint8_t* scales, const float* g, const int64_t* rs,
                             const int64_t* cs, int64_t count, double* y, double* d) {
  int64_t t;
  if (rows < 0 || n < 0 || k < 0 || (k % 16) != 0) return ORC_ERR_ARG;
  if (!offsets_valid(offsets, rows, E)) return ORC_ERR_ARG;
  for (t = 0; t < count; ++t)
    if (rs[t] < 0 || rs[t] >= rows || cs[t] < 0 || cs[t] >= n) return ORC_ERR_ARG;
#pragma omp parallel for schedule(dynamic, 16)
  for (t = 0; t < count; ++t) {
    int64_t e = 0;
    while (!(rs[t] >= offsets[e] && rs[t] < offsets[e + 1])) ++e;
    dot_row(x + rs[t] * k, packed + (e * n + cs[t]) * (k / 2),
            scales + (e * n + cs[t]) * (k / 16), k, g[e], &y[t], &d[t]);
  }
  return ORC_OK;
}
