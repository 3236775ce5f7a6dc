/* Driver of the CPU oracle for AddressSanitizer / UndefinedBehaviorSanitizer
 * builds: every oracle function on small seeded inputs (ragged lengths,
 * empty slots, several tokens, k = N), with simple checks of the results.
 * Built together with oracle.c; exit status 0 when every check holds. */
#include <math.h>
#include <stdint.h>
#include <stdio.h>
#include <stdlib.h>
#include <string.h>

void oracle_bf16_decode(const uint16_t* in, double* out, int64_t n);
void oracle_indexer(const uint16_t* q, const uint16_t* k, const float* w, float* s, int B, int N,
                    int H, int D);
void oracle_indexer_mt(const uint16_t* q, const uint16_t* k, const float* w, float* s, int B,
                       int T, int N, int H, int D);
int oracle_topk(const void* scores, int dtype, int B, int N, int k, int32_t* idx, int order);
int oracle_topk_ragged(const void* scores, int dtype, int B, int N, const int32_t* lengths, int k,
                       int32_t* idx, int order);
int oracle_attend(const uint16_t* q, const uint16_t* kv, const int32_t* idx, const uint16_t* win,
                  double* out, int B, int N, int k, int W, int Hq, int D, double scale);
int oracle_attend_sink(const uint16_t* q, const uint16_t* kv, const int32_t* idx,
                       const uint16_t* win, const double* sink, double* out, int B, int N, int k,
                       int W, int Hq, int D, double scale);
int oracle_attend_mt(const uint16_t* q, const uint16_t* kv, const int32_t* idx, const uint16_t* win,
                     double* out, int B, int T, int N, int k, int W, int Hq, int D, double scale);
int oracle_step(const uint16_t* q_idx, const uint16_t* k_idx, const float* w, const uint16_t* q,
                const uint16_t* kv, const uint16_t* win, float* scores, int32_t* idx, double* out,
                int B, int N, int H, int DI, int k, int W, int Hq, int D, double scale);
int oracle_step_ragged(const uint16_t* q_idx, const uint16_t* k_idx, const float* w,
                       const uint16_t* q, const uint16_t* kv, const uint16_t* win,
                       const int32_t* lengths, float* scores, int32_t* idx, double* out, int B,
                       int N, int H, int DI, int k, int W, int Hq, int D, double scale);
int oracle_step_mt(const uint16_t* q_idx, const uint16_t* k_idx, const float* w, const uint16_t* q,
                   const uint16_t* kv, const uint16_t* win, const int32_t* lengths, float* scores,
                   int32_t* idx, double* out, int B, int T, int N, int H, int DI, int k, int W,
                   int Hq, int D, double scale);
void oracle_qproj(const uint16_t* x, const uint16_t* w, double* out, int B, int d_in, int O);
void oracle_compress(const uint16_t* x, const float* wg, double* out, int B, int G, int D);

static uint32_t rng = 12345u;
static uint32_t next(void) { rng = rng * 1664525u + 1013904223u; return rng; }
/* A bf16 value in about [-2, 2): exponent 126..128, random mantissa and sign. */
static uint16_t rbf16(void) {
  uint32_t r = next();
  return (uint16_t)(((r >> 31) << 15) | ((126u + (r >> 8) % 3u) << 7) | (r & 0x7Fu));
}
static uint16_t* bf(size_t n) {
  uint16_t* p = malloc(n * sizeof *p);
  for (size_t i = 0; i < n; ++i) p[i] = rbf16();
  return p;
}
static int fails = 0;
#define CHECK(c) do { if (!(c)) { fprintf(stderr, "check failed: %s (line %d)\n", #c, __LINE__); ++fails; } } while (0)

static int distinct(const int32_t* v, int n, int N) {
  for (int i = 0; i < n; ++i) {
    if (v[i] < 0 || v[i] >= N) return 0;
    for (int j = 0; j < i; ++j) if (v[i] == v[j]) return 0;
  }
  return 1;
}

int main(void) {
  const int B = 2, T = 2, N = 67, H = 3, DI = 128, k = 9, W = 3, Hq = 16, D = 128;
  uint16_t *qi = bf((size_t)B * T * H * DI), *ki = bf((size_t)B * N * DI);
  uint16_t *q = bf((size_t)B * T * Hq * D), *kv = bf((size_t)B * N * D), *win = bf((size_t)B * T * W * D);
  float* w = malloc(sizeof(float) * B * T * H);
  for (int i = 0; i < B * T * H; ++i) w[i] = (float)(next() % 1000) / 1000.0f;
  float* s = malloc(sizeof(float) * B * T * N);
  int32_t* idx = malloc(sizeof(int32_t) * B * T * k);
  double* out = malloc(sizeof(double) * B * T * Hq * D);
  double dec[4];
  oracle_bf16_decode(qi, dec, 4);
  oracle_indexer(qi, ki, w, s, B, N, H, DI);
  for (int i = 0; i < B * N; ++i) CHECK(s[i] >= 0.0f);
  CHECK(oracle_topk(s, 1, B, N, k, idx, 0) == 0);
  for (int b = 0; b < B; ++b) CHECK(distinct(idx + b * k, k, N));
  CHECK(oracle_topk(s, 1, B, N, N, malloc(sizeof(int32_t) * B * N), 1) == 0);  /* k = N */
  CHECK(oracle_topk(s, 1, B, N, N + 1, idx, 0) == -1);
  const int32_t lengths[4] = {0, 5, N, 40};
  CHECK(oracle_topk_ragged(s, 1, B, N, lengths, k, idx, 1) == 0);
  CHECK(idx[0] == -1 && idx[k - 1] == -1);
  CHECK(oracle_attend(q, kv, idx, win, out, B, N, k, W, Hq, D, 0.1) == 0);
  for (int i = 0; i < B * Hq * D; ++i) CHECK(isfinite(out[i]));
  double sink[16];
  for (int h = 0; h < Hq; ++h) sink[h] = h == 0 ? -INFINITY : (double)h / 4.0;
  CHECK(oracle_attend_sink(q, kv, idx, win, sink, out, B, N, k, W, Hq, D, 0.1) == 0);
  CHECK(oracle_step(qi, ki, w, q, kv, win, s, idx, out, B, N, H, DI, k, W, Hq, D, 0.1) == 0);
  CHECK(oracle_step_ragged(qi, ki, w, q, kv, win, lengths, s, idx, out, B, N, H, DI, k, W, Hq, D,
                           0.1) == 0);
  oracle_indexer_mt(qi, ki, w, s, B, T, N, H, DI);
  CHECK(oracle_step_mt(qi, ki, w, q, kv, win, lengths, s, idx, out, B, T, N, H, DI, k, W, Hq, D,
                       0.1) == 0);
  CHECK(oracle_attend_mt(q, kv, idx, win, out, B, T, N, k, W, Hq, D, 0.1) == 0);
  const int bad[2] = {N, 0};
  CHECK(oracle_attend(q, kv, bad, win, out, 1, N, 1, 0, Hq, D, 0.1) == -1);
  double* pj = malloc(sizeof(double) * B * 256);
  oracle_qproj(kv, kv, pj, B, 128, 2);
  double* cmp = malloc(sizeof(double) * B * 3 * D);
  float* wg = malloc(sizeof(float) * D);
  for (int d = 0; d < D; ++d) wg[d] = (float)((int)(next() % 200) - 100) / 400.0f;
  uint16_t* raw = bf((size_t)B * 12 * D);
  oracle_compress(raw, wg, cmp, B, 3, D);
  for (int i = 0; i < B * 3 * D; ++i) CHECK(isfinite(cmp[i]));
  printf("oracle driver: %d failed checks\n", fails);
  return fails ? 1 : 0;
}
