/* driver.c -- runs every C entry point of the CPU oracle (oracle/
 * nvfp4_oracle.c, compiled into the same executable) on small inputs that
 * reach its edge cases, so that the test can build it with AddressSanitizer
 * and UndefinedBehaviorSanitizer and see no report.  Exit status 0 when
 * every call returned what it should. */
#include <math.h>
#include <stdint.h>
#include <stdio.h>
#include <stdlib.h>
#include <string.h>

double orc_e2m1_value(unsigned code);
double orc_e4m3_value(unsigned code);
uint8_t orc_e4m3_encode(float x);
uint8_t orc_e2m1_encode_mag(float q);
void orc_e4m3_encode_array(const float* x, int64_t n, uint8_t* out);
void orc_e2m1_encode_mag_array(const float* q, int64_t n, uint8_t* out);
float orc_global_scale(float amax);
uint8_t orc_block_scale_code(float amax_b, float g);
uint8_t orc_element_code(float w, float s_dec, float g);
int orc_quantize(const uint16_t* w, int64_t batch, int64_t n, int64_t k, uint8_t* packed,
                 uint8_t* scales, float* g_out);
void orc_dequant(const uint8_t* packed, const uint8_t* scales, int64_t n, int64_t k,
                 double* w_dec);
int orc_gemm(const uint16_t* x, int64_t m, int64_t n, int64_t k, const uint8_t* packed,
             const uint8_t* scales, float g, double* y, double* d);
int orc_gemm_sampled(const uint16_t* x, int64_t m, int64_t n, int64_t k, const uint8_t* packed,
                     const uint8_t* scales, float g, const int64_t* rows, const int64_t* cols,
                     int64_t count, double* y, double* d);
int orc_grouped_gemm(const uint16_t* x, int64_t rows, const int32_t* offsets, int64_t E,
                     int64_t n, int64_t k, const uint8_t* packed, const uint8_t* scales,
                     const float* g, double* y, double* d);
int orc_grouped_gemm_sampled(const uint16_t* x, int64_t rows, const int32_t* offsets,
                             int64_t E, int64_t n, int64_t k, const uint8_t* packed,
                             const uint8_t* scales, const float* g, const int64_t* rs,
                             const int64_t* cs, int64_t count, double* y, double* d);

#define CHECK(c)                                               \
  do {                                                         \
    if (!(c)) {                                                \
      fprintf(stderr, "check failed line %d: %s\n", __LINE__, #c); \
      return 1;                                                \
    }                                                          \
  } while (0)

static uint32_t state = 12345u;
static uint32_t next(void) {  /* xorshift32 */
  state ^= state << 13;
  state ^= state >> 17;
  state ^= state << 5;
  return state;
}

int main(void) {
  enum { B = 3, N = 20, K = 48, M = 7, E = 4 };
  static uint16_t w[B * N * K], x[M * K];
  static uint8_t packed[B * N * K / 2], scales[B * N * K / 16];
  static float g[B];
  static double wd[N * K], y[M * N], d[M * N];
  unsigned c;
  int64_t i;
  float qs[] = {0.0f, 0.25f, 0.75f, 1.25f, 1.75f, 2.5f, 3.5f, 5.0f, 6.0f, 7.0f, 1e30f, INFINITY};
  uint8_t out[64];

  for (c = 0; c < 16; ++c) (void)orc_e2m1_value(c);
  for (c = 0; c < 256; ++c) (void)orc_e4m3_value(c);
  CHECK(orc_e4m3_encode(448.0f) == 0x7E && orc_e4m3_encode(1e9f) == 0x7E);
  CHECK(orc_e2m1_encode_mag(6.0f) == 7 && orc_e2m1_encode_mag(0.25f) == 0);
  orc_e2m1_encode_mag_array(qs, 12, out);
  orc_e4m3_encode_array(qs, 10, out);
  CHECK(orc_global_scale(2688.0f) == 1.0f);
  CHECK(orc_block_scale_code(6.0f, 0.0f) == 0);
  CHECK((orc_element_code(-0.0f, 1.0f, 1.0f) & 8u) != 0);
  CHECK(orc_element_code(1.0f, 0.0f, 1.0f) == 0);

  /* three tensors: random normals' bits, subnormals and zeros, rounding ties */
  for (i = 0; i < N * K; ++i) w[i] = (uint16_t)(0x3C00u + (next() & 0x07FFu) + ((next() & 1u) << 15));
  for (i = 0; i < N * K; ++i) w[N * K + i] = (uint16_t)((next() & 0x01FFu) | ((next() & 1u) << 15));
  for (i = 0; i < N * K; ++i) w[2 * N * K + i] = (i % 5 == 0) ? 0x8000u : (uint16_t)(0x3E80u + (i % 7) * 0x40u);
  CHECK(orc_quantize(w, B, N, K, packed, scales, g) == 0);
  orc_dequant(packed, scales, N, K, wd);
  for (i = 0; i < M * K; ++i) x[i] = (uint16_t)(0x3F00u + (next() & 0x00FFu) + ((next() & 1u) << 15));
  CHECK(orc_gemm(x, M, N, K, packed, scales, g[0], y, d) == 0);
  CHECK(orc_gemm(x, 0, N, K, packed, scales, g[0], y, d) == 0);
  CHECK(orc_gemm(x, M, N, 40 + 1, packed, scales, g[0], y, d) != 0);  /* k % 16 != 0 */
  {
    int64_t rows[] = {0, M - 1, 3}, cols[] = {N - 1, 0, 5}, bad[] = {M, 0, 0};
    CHECK(orc_gemm_sampled(x, M, N, K, packed, scales, g[0], rows, cols, 3, y, d) == 0);
    CHECK(orc_gemm_sampled(x, M, N, K, packed, scales, g[0], bad, cols, 3, y, d) != 0);
  }
  {
    int32_t off[E + 1] = {0, 2, 2, 6, M};  /* one empty expert */
    int32_t bad_off[E + 1] = {0, 3, 2, 6, M};
    float ge[E] = {g[0], g[1], g[2], g[0]};
    static uint8_t pe[E * N * K / 2], se[E * N * K / 16];
    int64_t rs[] = {0, 2, 5, 6}, cs[] = {1, 2, 3, N - 1};
    memcpy(pe, packed, sizeof(packed));
    memcpy(pe + B * N * K / 2, packed, N * K / 2);
    memcpy(se, scales, sizeof(scales));
    memcpy(se + B * N * K / 16, scales, N * K / 16);
    CHECK(orc_grouped_gemm(x, M, off, E, N, K, pe, se, ge, y, d) == 0);
    CHECK(orc_grouped_gemm(x, M, bad_off, E, N, K, pe, se, ge, y, d) != 0);
    CHECK(orc_grouped_gemm_sampled(x, M, off, E, N, K, pe, se, ge, rs, cs, 4, y, d) == 0);
  }
  /* a non-finite weight is reported */
  w[5] = 0x7F80u;
  CHECK(orc_quantize(w, 1, N, K, packed, scales, g) != 0);
  printf("oracle driver ok\n");
  return 0;
}
