/*
 * CPU oracle for the sparse-attention decode step.
 *
 * TEST INFRASTRUCTURE ONLY. This file is the plain, slow, obviously correct
 * definition that the GPU library is checked against. Nothing in the GPU
 * library includes, links or calls it; only the tests, the smoke check and
 * the CPU-baseline leg of the benchmark load it. It shares no code, header,
 * table or helper with the HIP sources.
 *
 * Sources (cited by page title and section):
 *  [CSA]  "feat: Add DeepSeek-V4 CSA attention kernels" (aws-neuron
 *         nki-library pull request 13), section "How the algorithm works",
 *         the step table (steps 2, 3, 4), and the paragraph after the GpSimd
 *         bullet list (keys and values are one tensor).
 *  [DS]   "DeepSelect" project page (deepseek-ai/DeepSelect), the algorithm
 *         and scenario paragraphs (top-k by score, sorted_index and
 *         return_value options).
 *  [PTB]  "Implementation: Deepspeedai DeepSpeed Inference PT Binding",
 *         Usage Examples (norm_factor = 1/sqrt(head_dim) scales q.k).
 *
 * Readings where the pages are silent (each is listed in the design notes):
 *  - indexer: ReLU is applied per head to the q.k product, then the result is
 *    multiplied by that head's weight, then summed over heads; no other scale.
 *  - scores are accumulated in double and rounded once to float.
 *  - top-k order: value descending, ties broken by lower index; -0 == +0.
 *  - attention: rows = selected compressed rows followed by the W window
 *    rows; the same row serves as key and value; plain softmax, no mask.
 *  - ragged rows (an extension): row b has lengths[b] valid positions; its
 *    top-k slots past min(k, lengths[b]) hold -1, and a -1 slot takes no
 *    part in attention (a batch row with no rows gets zeros).
 *  - indexer query projection: a plain matrix-vector product per batch row
 *    (the projection weights are synthetic; the pages give no widths).
 *  - several query tokens per batch row (an extension): T consecutive query
 *    rows share one row of keys (indexer keys and compressed KV); each has
 *    its own queries, weights, window, length and selection, and is in
 *    every other respect an independent decode row.
 *  - attention sink: one logit per query head, in the units of the scaled
 *    q.k logits, that takes part in the softmax normalisation like a row
 *    whose value vector is zero (so it adds to the denominator only).
 *  - compressor: each group of 4 consecutive raw KV rows becomes one
 *    compressed row, the softmax (over the 4 rows) of a linear gate score
 *    of each row weighting the rows' sum.
 *
 * Every floating-point step runs in double. bf16 inputs are decoded exactly.
 * OpenMP, when enabled, only splits independent batch rows; the result does
 * not depend on the thread count.
 */
#include <math.h>
#include <stdint.h>
#include <stdlib.h>
#include <string.h>
#ifdef _OPENMP
#include <omp.h>
#endif

/* Thread count for the row-parallel loops (1 when built without OpenMP). */
void oracle_set_threads(int n) {
#ifdef _OPENMP
  if (n > 0) omp_set_num_threads(n);
#else
  (void)n;
#endif
}

int oracle_max_threads(void) {
#ifdef _OPENMP
  return omp_get_max_threads();
#else
  return 1;
#endif
}

/* bf16 is the top half of an IEEE binary32: widening is exact. */
static double bf16_value(uint16_t bits) {
  uint32_t w = (uint32_t)bits << 16;
  float f;
  memcpy(&f, &w, sizeof f);
  return (double)f;
}

void oracle_bf16_decode(const uint16_t* in, double* out, int64_t n) {
  for (int64_t i = 0; i < n; ++i) out[i] = bf16_value(in[i]);
}

/*
 * Lightning-indexer score [CSA, step 2]:
 *   s[b,j] = sum_h w[b,h] * max(0, sum_d q[b,h,d] * k[b,j,d])
 * q: bf16 [B,H,D], k: bf16 [B,N,D], w: float [B,H], s: float [B,N].
 */
static void indexer_rows(const uint16_t* q, const uint16_t* k, const float* w,
                         float* s, int B, int T, int N, int H, int D) {
  /* query row b reads the keys of batch row b / T */
#pragma omp parallel for schedule(static)
  for (int b = 0; b < B * T; ++b) {
    for (int j = 0; j < N; ++j) {
      const uint16_t* krow = k + ((int64_t)(b / T) * N + j) * D;
      double total = 0.0;
      for (int h = 0; h < H; ++h) {
        const uint16_t* qrow = q + ((int64_t)b * H + h) * D;
        double dot = 0.0;
        for (int d = 0; d < D; ++d) dot += bf16_value(qrow[d]) * bf16_value(krow[d]);
        double relu = dot > 0.0 ? dot : 0.0;
        total += (double)w[(int64_t)b * H + h] * relu;
      }
      s[(int64_t)b * N + j] = (float)total;
    }
  }
}

void oracle_indexer(const uint16_t* q, const uint16_t* k, const float* w,
                    float* s, int B, int N, int H, int D) {
  indexer_rows(q, k, w, s, B, 1, N, H, D);
}

/* T query tokens per batch row: q bf16 [B*T,H,D], w [B*T,H], s [B*T,N];
 * k bf16 [B,N,D] is shared by the T tokens of a row. */
void oracle_indexer_mt(const uint16_t* q, const uint16_t* k, const float* w,
                       float* s, int B, int T, int N, int H, int D) {
  indexer_rows(q, k, w, s, B, T, N, H, D);
}

/*
 * Top-k [CSA step 3; DS]: the k positions with the largest score. The order
 * used is the one a stable sort by descending value gives: a larger value
 * comes first, and of two equal values the lower index comes first. The
 * comparison is between IEEE values, so -0.0 and +0.0 are equal.
 */
typedef struct {
  double v;
  int32_t i;
} keyed_t;

static int by_value_desc_then_index(const void* pa, const void* pb) {
  const keyed_t* a = (const keyed_t*)pa;
  const keyed_t* b = (const keyed_t*)pb;
  if (a->v > b->v) return -1;
  if (a->v < b->v) return 1;
  return (a->i > b->i) - (a->i < b->i);
}

static int by_index(const void* pa, const void* pb) {
  int32_t a = *(const int32_t*)pa, b = *(const int32_t*)pb;
  return (a > b) - (a < b);
}

/* One row: vals[N] (already decoded) -> idx[k]. index_order: 0 gives the
 * (value desc, index asc) order, 1 gives ascending index order. */
static void topk_row(const double* vals, int N, int k, int32_t* idx,
                     int index_order, keyed_t* tmp) {
  for (int j = 0; j < N; ++j) {
    tmp[j].v = vals[j];
    tmp[j].i = j;
  }
  qsort(tmp, (size_t)N, sizeof(keyed_t), by_value_desc_then_index);
  for (int t = 0; t < k; ++t) idx[t] = tmp[t].i;
  if (index_order) qsort(idx, (size_t)k, sizeof(int32_t), by_index);
}

/* dtype: 0 = bf16 bits (uint16), 1 = float32. Returns 0, or -1 on bad args. */
int oracle_topk(const void* scores, int dtype, int B, int N, int k,
                int32_t* idx, int index_order) {
  if (B < 1 || N < 1 || k < 1 || k > N || (dtype != 0 && dtype != 1)) return -1;
  int bad = 0;
#pragma omp parallel
  {
    double* vals = (double*)malloc(sizeof(double) * (size_t)N);
    keyed_t* tmp = (keyed_t*)malloc(sizeof(keyed_t) * (size_t)N);
    if (!vals || !tmp) {
#pragma omp atomic write
      bad = 1;
    } else {
#pragma omp for schedule(static)
      for (int b = 0; b < B; ++b) {
        for (int j = 0; j < N; ++j) {
          int64_t at = (int64_t)b * N + j;
          vals[j] = dtype == 0 ? bf16_value(((const uint16_t*)scores)[at])
                               : (double)((const float*)scores)[at];
        }
        topk_row(vals, N, k, idx + (int64_t)b * k, index_order, tmp);
      }
    }
    free(vals);
    free(tmp);
  }
  return bad ? -1 : 0;
}

/*
 * Ragged rows (a reading beyond [CSA], whose block takes one compressed
 * length T_c for the whole batch in its launch listing, with the sequence
 * length a driver option): in a serving batch each sequence has its own
 * length, so row b holds lengths[b] valid positions (0 <= lengths[b] <= N;
 * later positions take no part). Its first min(k, lengths[b]) output slots
 * hold the top-k of the valid prefix, in the same order as oracle_topk, and
 * the remaining slots hold -1. Returns 0, or -1 on bad args.
 */
int oracle_topk_ragged(const void* scores, int dtype, int B, int N, const int32_t* lengths,
                       int k, int32_t* idx, int index_order) {
  if (B < 1 || N < 1 || k < 1 || k > N || (dtype != 0 && dtype != 1)) return -1;
  for (int b = 0; b < B; ++b)
    if (lengths[b] < 0 || lengths[b] > N) return -1;
  int bad = 0;
#pragma omp parallel
  {
    double* vals = (double*)malloc(sizeof(double) * (size_t)N);
    keyed_t* tmp = (keyed_t*)malloc(sizeof(keyed_t) * (size_t)N);
    if (!vals || !tmp) {
#pragma omp atomic write
      bad = 1;
    } else {
#pragma omp for schedule(static)
      for (int b = 0; b < B; ++b) {
        const int n = lengths[b];
        const int kk = k < n ? k : n;
        int32_t* out = idx + (int64_t)b * k;
        for (int j = 0; j < n; ++j) {
          int64_t at = (int64_t)b * N + j;
          vals[j] = dtype == 0 ? bf16_value(((const uint16_t*)scores)[at])
                               : (double)((const float*)scores)[at];
        }
        if (kk > 0) topk_row(vals, n, kk, out, index_order, tmp);
        for (int t = kk; t < k; ++t) out[t] = -1;
      }
    }
    free(vals);
    free(tmp);
  }
  return bad ? -1 : 0;
}

/*
 * Sparse multi-query attention for one decode token [CSA step 4; PTB]:
 *   R_b = rows kv[b, idx[b,0..k)] followed by rows win[b, 0..W)
 *   z[h,r] = scale * q[b,h,:] . R_b[r,:]
 *   p[h,:] = softmax over r of z[h,:]
 *   out[b,h,:] = sum_r p[h,r] * R_b[r,:]          (the row is key and value)
 * q: bf16 [B,Hq,D]; kv: bf16 [B,N,D]; idx: int32 [B,k] with values in [0,N),
 * or -1 for a slot that holds no row (ragged rows: it takes no part);
 * win: bf16 [B,W,D] (unused when W == 0); out: double [B,Hq,D]. A batch row
 * with no rows at all gets a zero output.
 * Returns 0, or -1 if an index is out of range.
 */
static int attend_rows(const uint16_t* q, const uint16_t* kv, const int32_t* idx,
                       const uint16_t* win, const double* sink, double* out, int B, int T,
                       int N, int k, int W, int Hq, int D, double scale) {
  /* query row b gathers from the compressed rows of batch row b / T */
  for (int64_t t = 0; t < (int64_t)B * T * k; ++t)
    if (idx[t] < -1 || idx[t] >= N) return -1;
  const int R = k + W;
  if (R < 1) return -1;
#pragma omp parallel
  {
    double* rows = (double*)malloc(sizeof(double) * (size_t)R * (size_t)D);
    double* z = (double*)malloc(sizeof(double) * (size_t)R);
    double* qd = (double*)malloc(sizeof(double) * (size_t)D);
#pragma omp for schedule(static)
    for (int b = 0; b < B * T; ++b) {
      int nr = 0;  /* rows that take part, gathered in slot order */
      for (int r = 0; r < R; ++r) {
        if (r < k && idx[(int64_t)b * k + r] < 0) continue;
        const uint16_t* src =
            r < k ? kv + ((int64_t)(b / T) * N + idx[(int64_t)b * k + r]) * D
                  : win + ((int64_t)b * W + (r - k)) * D;
        for (int d = 0; d < D; ++d) rows[(int64_t)nr * D + d] = bf16_value(src[d]);
        ++nr;
      }
      for (int h = 0; h < Hq; ++h) {
        const uint16_t* qrow = q + ((int64_t)b * Hq + h) * D;
        for (int d = 0; d < D; ++d) qd[d] = bf16_value(qrow[d]);
        double* o = out + ((int64_t)b * Hq + h) * D;
        if (nr == 0) {
          for (int d = 0; d < D; ++d) o[d] = 0.0;
          continue;
        }
        /* The sink (when given) competes for the maximum and adds exp(sink - m)
         * to the denominator; it brings no value vector. */
        double m = sink ? sink[h] : -INFINITY;
        for (int r = 0; r < nr; ++r) {
          double dot = 0.0;
          for (int d = 0; d < D; ++d) dot += qd[d] * rows[(int64_t)r * D + d];
          z[r] = scale * dot;
          if (z[r] > m) m = z[r];
        }
        double l = sink ? exp(sink[h] - m) : 0.0;
        for (int r = 0; r < nr; ++r) {
          z[r] = exp(z[r] - m);
          l += z[r];
        }
        for (int d = 0; d < D; ++d) {
          double acc = 0.0;
          for (int r = 0; r < nr; ++r) acc += z[r] * rows[(int64_t)r * D + d];
          o[d] = acc / l;
        }
      }
    }
    free(rows);
    free(z);
    free(qd);
  }
  return 0;
}

int oracle_attend(const uint16_t* q, const uint16_t* kv, const int32_t* idx,
                  const uint16_t* win, double* out, int B, int N, int k, int W,
                  int Hq, int D, double scale) {
  return attend_rows(q, kv, idx, win, NULL, out, B, 1, N, k, W, Hq, D, scale);
}

/*
 * Attention with a sink [CSA, "DMA Traffic Shaping", priority table, where
 * the attention sink is one of the transfers of the attention kernel; the
 * pages give no formula, so this is a reading]: sink[h] (double [Hq], finite
 * or -inf) is a logit of head h, in the units of z, that joins the softmax
 * normalisation and brings no value vector:
 *   m = max(sink[h], max_r z[h,r])
 *   out[b,h,:] = sum_r exp(z[h,r] - m) R_b[r,:] / (exp(sink[h] - m) + sum_r exp(z[h,r] - m))
 * sink[h] = -inf gives plain attention. A batch row with no rows at all
 * still gets a zero output.
 */
int oracle_attend_sink(const uint16_t* q, const uint16_t* kv, const int32_t* idx,
                       const uint16_t* win, const double* sink, double* out, int B, int N,
                       int k, int W, int Hq, int D, double scale) {
  return attend_rows(q, kv, idx, win, sink, out, B, 1, N, k, W, Hq, D, scale);
}

/* T query tokens per batch row: q [B*T,Hq,D], idx [B*T,k], win [B*T,W,D],
 * out [B*T,Hq,D]; kv [B,N,D] is shared by the T tokens of a row. */
int oracle_attend_mt(const uint16_t* q, const uint16_t* kv, const int32_t* idx,
                     const uint16_t* win, double* out, int B, int T, int N, int k,
                     int W, int Hq, int D, double scale) {
  return attend_rows(q, kv, idx, win, NULL, out, B, T, N, k, W, Hq, D, scale);
}

/*
 * The whole decode step [CSA, steps 2 -> 3 -> 4]: indexer scores, then the
 * top-k of each score row, then attention over the selected rows plus the
 * window. scores [B,N] and idx [B,k] (value-desc order) are outputs too.
 */
int oracle_step(const uint16_t* q_idx, const uint16_t* k_idx, const float* w,
                const uint16_t* q, const uint16_t* kv, const uint16_t* win,
                float* scores, int32_t* idx, double* out, int B, int N, int H,
                int DI, int k, int W, int Hq, int D, double scale) {
  oracle_indexer(q_idx, k_idx, w, scores, B, N, H, DI);
  if (oracle_topk(scores, 1, B, N, k, idx, 0) != 0) return -1;
  return oracle_attend(q, kv, idx, win, out, B, N, k, W, Hq, D, scale);
}

/* The same step over ragged rows: the top-k of row b looks only at its
 * first lengths[b] scores, and empty slots (-1) take no part in attention. */
int oracle_step_ragged(const uint16_t* q_idx, const uint16_t* k_idx, const float* w,
                       const uint16_t* q, const uint16_t* kv, const uint16_t* win,
                       const int32_t* lengths, float* scores, int32_t* idx, double* out,
                       int B, int N, int H, int DI, int k, int W, int Hq, int D,
                       double scale) {
  oracle_indexer(q_idx, k_idx, w, scores, B, N, H, DI);
  if (oracle_topk_ragged(scores, 1, B, N, lengths, k, idx, 0) != 0) return -1;
  return oracle_attend(q, kv, idx, win, out, B, N, k, W, Hq, D, scale);
}

/* The step with T query tokens per batch row: the indexer scores every
 * token against its row's keys, each token's score row gets its own top-k
 * (over its first lengths[b*T+t] positions when lengths is given, else all
 * N), and each token attends over its own selection and window. */
int oracle_step_mt(const uint16_t* q_idx, const uint16_t* k_idx, const float* w,
                   const uint16_t* q, const uint16_t* kv, const uint16_t* win,
                   const int32_t* lengths, float* scores, int32_t* idx, double* out,
                   int B, int T, int N, int H, int DI, int k, int W, int Hq, int D,
                   double scale) {
  if (T < 1) return -1;
  oracle_indexer_mt(q_idx, k_idx, w, scores, B, T, N, H, DI);
  const int rc = lengths ? oracle_topk_ragged(scores, 1, B * T, N, lengths, k, idx, 0)
                         : oracle_topk(scores, 1, B * T, N, k, idx, 0);
  if (rc != 0) return -1;
  return oracle_attend_mt(q, kv, idx, win, out, B, T, N, k, W, Hq, D, scale);
}

/*
 * Indexer query projection [CSA, step table, step 2: the indexer query is
 * projected into 128 channels per head before scoring]:
 *   out[b, o] = sum_i x[b, i] * w[o, i]
 * x bf16 [B, d_in], w bf16 [O, d_in] (O = H_I * 128 output channels, row o
 * of w holding output o's weights), out double [B, O]. Products of bf16
 * values are exact in double; the sum runs in double in index order.
 */
void oracle_qproj(const uint16_t* x, const uint16_t* w, double* out, int B, int d_in, int O) {
#pragma omp parallel for schedule(static)
  for (int o = 0; o < O; ++o) {
    const uint16_t* wrow = w + (int64_t)o * d_in;
    for (int b = 0; b < B; ++b) {
      const uint16_t* xrow = x + (int64_t)b * d_in;
      double acc = 0.0;
      for (int i = 0; i < d_in; ++i) acc += bf16_value(xrow[i]) * bf16_value(wrow[i]);
      out[(int64_t)b * O + o] = acc;
    }
  }
}

/*
 * Compressor [CSA, "How the algorithm works", step table, step 1: every 4
 * raw tokens are folded into one compressed entry by a gated weighted sum].
 * The pages give no formula; reading: each raw KV row x_i (i < 4 of one
 * group) gets a gate score z_i = sum_d wg[d] * x_i[d] (one learned gate
 * vector wg), the weights are the softmax of the 4 scores, and the
 * compressed row is the weighted sum:
 *   a_i = exp(z_i - max_j z_j) / sum_j exp(z_j - max_j z_j)
 *   out[b, g, d] = sum_i a_i * x[b, 4g + i, d]
 * x bf16 [B, 4G, D] (raw rows, group g = rows 4g .. 4g+3), wg float [D], out
 * double [B, G, D]. Every step runs in double.
 */
void oracle_compress(const uint16_t* x, const float* wg, double* out, int B, int G, int D) {
#pragma omp parallel for schedule(static)
  for (int bg = 0; bg < B * G; ++bg) {
    const uint16_t* rows = x + (int64_t)bg * 4 * D;  /* group bg's 4 rows are consecutive */
    double z[4], a[4];
    double zmax = -INFINITY;
    for (int i = 0; i < 4; ++i) {
      double dot = 0.0;
      for (int d = 0; d < D; ++d) dot += (double)wg[d] * bf16_value(rows[(int64_t)i * D + d]);
      z[i] = dot;
      if (dot > zmax) zmax = dot;
    }
    double l = 0.0;
    for (int i = 0; i < 4; ++i) {
      a[i] = exp(z[i] - zmax);
      l += a[i];
    }
    double* o = out + (int64_t)bg * D;
    for (int d = 0; d < D; ++d) {
      double acc = 0.0;
      for (int i = 0; i < 4; ++i) acc += (a[i] / l) * bf16_value(rows[(int64_t)i * D + d]);
      o[d] = acc;
    }
  }
}
