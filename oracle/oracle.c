/*
 * oracle.c -- plain, slow, FP64 CPU oracle for block-scaled 4-bit and FP8 decode
 * matrix-vector products.
 *
 * TEST INFRASTRUCTURE ONLY.  Only tests/, __graft_entry__.smoke() and the
 * cpu_baseline leg of bench.py may load or call this code.  It shares no code,
 * header, table or constant with the GPU library, and the GPU library never
 * calls it.
 *
 * What it computes (all arithmetic in double, sequential sums, no blocking):
 *
 *  - Weight decode.  "Decode speed is bytes divided by bandwidth" / "Fewer bytes
 *    per weight: NVFP4" (page: mdjawad.com, DGX Spark tag feed) describe NVFP4 as
 *    E2M1 elements (1 sign, 2 exponent, 1 mantissa bit; values 0, +-0.5, +-1,
 *    +-1.5, +-2, +-3, +-4, +-6), one E4M3 scale per 16 consecutive weights and one
 *    FP32 scale per tensor.  The reconstruction formula itself was lost in the
 *    page's extraction; the reading taken here is w = e2m1 * block_scale *
 *    tensor_scale.  MXFP4 (page: magicnetworld.com Ling-3.0 article, sec. 3 and
 *    the glossary, which calls it a 4-bit micro-scaling float whose scale is
 *    shared by a small block and leaves the block size open) is read
 *    as E2M1 elements with one E8M0 power-of-two scale per 32 weights.  The FP8
 *    output layer (same article, sec. 7; mdjawad.com feed, "Fewer bytes per
 *    weight") is read as OCP E4M3FN codes with one FP32 scale per row.
 *
 *  - The product.  A matrix with d_out rows and d_in columns maps a length-d_in
 *    vector to a length-d_out one with one multiply and one add per weight
 *    (mdjawad.com feed, "Decode speed is bytes divided by bandwidth"):
 *    y[r] = sum_k w[r][k] * x[k].  The verify pass of speculative decoding
 *    multiplies each matrix by K+1 vectors (same feed, "More tokens per weight
 *    read"), so every routine takes M input vectors.
 *
 *  - Tolerance helper.  A[r] = sum_k |w[r][k] * x[k]|, the scale against which
 *    GPU results are compared.
 *
 *  - MoE routing (magicnetworld.com article, sec. 3 and sec. 4 flowchart: each
 *    token goes to 8 of 512 routed experts plus 1 shared expert): top-k by logit
 *    (descending, ties to the lower index) and a softmax over the k selected
 *    logits.
 *
 *  - SiLU(z) = z / (1 + exp(-z)).
 *
 * Logical (unpacked) operand layouts, row-major:
 *   NVFP4  : codes u8[d_out][d_in/2]  (byte j holds column 2j in bits 0-3 and
 *            column 2j+1 in bits 4-7), scales u8[d_out][d_in/16] (E4M3FN),
 *            plus one tensor scale.
 *   MXFP4  : codes as NVFP4, scales u8[d_out][d_in/32] (E8M0).
 *   FP8ROW : codes u8[d_out][d_in] (E4M3FN), scales f32[d_out].
 *   X      : bf16 bit patterns u16[M][d_in].
 */
#include <math.h>
#include <pthread.h>
#include <stdint.h>
#include <stdlib.h>
#include <string.h>

#define OR_NVFP4 1
#define OR_MXFP4 2
#define OR_FP8ROW 3

/* E2M1: bit 3 sign, bits 2-1 exponent (bias 1), bit 0 mantissa.  Exponent 0 is
 * the subnormal case: 0 or 0.5. */
double or_e2m1(unsigned code) {
  unsigned s = (code >> 3) & 1u, e = (code >> 1) & 3u, m = code & 1u;
  double mag = (e == 0) ? 0.5 * (double)m : ldexp(1.0 + 0.5 * (double)m, (int)e - 1);
  return s ? -mag : mag;
}

/* OCP E4M3FN: bit 7 sign, bits 6-3 exponent (bias 7), bits 2-0 mantissa; no
 * infinities; S.1111.111 is NaN. */
double or_e4m3(unsigned b) {
  unsigned s = (b >> 7) & 1u, e = (b >> 3) & 15u, m = b & 7u;
  double mag;
  if (e == 15 && m == 7) return NAN;
  if (e == 0)
    mag = ldexp((double)m / 8.0, -6);
  else
    mag = ldexp(1.0 + (double)m / 8.0, (int)e - 7);
  return s ? -mag : mag;
}

/* E8M0: an unsigned biased exponent, 2^(b-127); 0xFF is NaN. */
double or_e8m0(unsigned b) {
  if ((b & 255u) == 255u) return NAN;
  return ldexp(1.0, (int)(b & 255u) - 127);
}

/* bfloat16: the upper 16 bits of an IEEE binary32. */
double or_bf16(uint16_t h) {
  uint32_t u = (uint32_t)h << 16;
  float f;
  memcpy(&f, &u, sizeof f);
  return (double)f;
}

double or_silu(double z) { return z / (1.0 + exp(-z)); }

/* One dequantised weight w[r][k], straight from the definition. */
static double weight(int fmt, int64_t d_in, const uint8_t* codes, const void* scales,
                     double tensor_scale, int64_t r, int64_t k) {
  if (fmt == OR_FP8ROW) {
    const float* rs = (const float*)scales;
    return or_e4m3(codes[r * d_in + k]) * (double)rs[r];
  }
  uint8_t byte = codes[r * (d_in / 2) + k / 2];
  unsigned nib = (k & 1) ? (byte >> 4) : (byte & 15u);
  const uint8_t* sc = (const uint8_t*)scales;
  if (fmt == OR_NVFP4) return or_e2m1(nib) * or_e4m3(sc[r * (d_in / 16) + k / 16]) * tensor_scale;
  return or_e2m1(nib) * or_e8m0(sc[r * (d_in / 32) + k / 32]);
}

typedef struct {
  int fmt, M;
  int64_t d_out, d_in, nrows, r0, r1;
  const uint8_t* codes;
  const void* scales;
  double tensor_scale;
  const uint16_t* X;
  const double* XD;
  const int64_t* rows;
  double *Y, *A;
} gemv_job;

static void* gemv_worker(void* p) {
  gemv_job* j = (gemv_job*)p;
  for (int64_t i = j->r0; i < j->r1; ++i) {
    int64_t r = j->rows ? j->rows[i] : i;
    for (int m = 0; m < j->M; ++m) {
      double y = 0.0, a = 0.0;
      for (int64_t k = 0; k < j->d_in; ++k) {
        double w = weight(j->fmt, j->d_in, j->codes, j->scales, j->tensor_scale, r, k);
        int64_t xi = (int64_t)m * j->d_in + k;
        double t = w * (j->XD ? j->XD[xi] : or_bf16(j->X[xi]));
        y += t;
        a += fabs(t);
      }
      j->Y[(int64_t)m * j->nrows + i] = y;
      if (j->A) j->A[(int64_t)m * j->nrows + i] = a;
    }
  }
  return NULL;
}

static int gemv_any(int fmt, int64_t d_out, int64_t d_in, const uint8_t* codes,
                    const void* scales, double tensor_scale, int M, const uint16_t* X,
                    const double* XD, const int64_t* rows, int64_t nrows, double* Y, double* A,
                    int nthreads) {
  if (fmt < OR_NVFP4 || fmt > OR_FP8ROW || M < 1 || d_out < 1 || d_in < 1) return -1;
  if (fmt == OR_NVFP4 && d_in % 16) return -1;
  if (fmt == OR_MXFP4 && d_in % 32) return -1;
  if (!rows && nrows != d_out) return -1;
  if (rows)
    for (int64_t i = 0; i < nrows; ++i)
      if (rows[i] < 0 || rows[i] >= d_out) return -1;
  if (nthreads < 1) nthreads = 1;
  if (nthreads > 256) nthreads = 256;
  if (nthreads > nrows) nthreads = (int)(nrows > 0 ? nrows : 1);
  gemv_job jobs[256];
  pthread_t th[256];
  for (int t = 0; t < nthreads; ++t) {
    gemv_job* j = &jobs[t];
    j->fmt = fmt; j->M = M; j->d_out = d_out; j->d_in = d_in; j->nrows = nrows;
    j->r0 = nrows * t / nthreads; j->r1 = nrows * (t + 1) / nthreads;
    j->codes = codes; j->scales = scales; j->tensor_scale = tensor_scale;
    j->X = X; j->XD = XD; j->rows = rows; j->Y = Y; j->A = A;
  }
  if (nthreads == 1) {
    gemv_worker(&jobs[0]);
    return 0;
  }
  for (int t = 0; t < nthreads; ++t) pthread_create(&th[t], NULL, gemv_worker, &jobs[t]);
  for (int t = 0; t < nthreads; ++t) pthread_join(th[t], NULL);
  return 0;
}

/* y[m][i] = sum_k w[rows[i]][k] * x[m][k]  and  A[m][i] = sum_k |w x|, with x
 * given as bf16 bit patterns X[M][d_in].  rows == NULL means all d_out rows
 * (nrows must then equal d_out).  Y and A are [M][nrows]; A may be NULL.
 * Returns 0 on success, -1 on a bad argument. */
int or_gemv(int fmt, int64_t d_out, int64_t d_in, const uint8_t* codes, const void* scales,
            double tensor_scale, int M, const uint16_t* X, const int64_t* rows, int64_t nrows,
            double* Y, double* A, int nthreads) {
  return gemv_any(fmt, d_out, d_in, codes, scales, tensor_scale, M, X, NULL, rows, nrows, Y, A,
                  nthreads);
}

/* The same product with x given in double, XD[M][d_in]. */
int or_gemv_dx(int fmt, int64_t d_out, int64_t d_in, const uint8_t* codes, const void* scales,
               double tensor_scale, int M, const double* XD, const int64_t* rows, int64_t nrows,
               double* Y, double* A, int nthreads) {
  return gemv_any(fmt, d_out, d_in, codes, scales, tensor_scale, M, NULL, XD, rows, nrows, Y, A,
                  nthreads);
}

/* Dequantise the whole logical matrix into W[d_out][d_in] (double). */
int or_dequant(int fmt, int64_t d_out, int64_t d_in, const uint8_t* codes, const void* scales,
               double tensor_scale, double* W) {
  if (fmt < OR_NVFP4 || fmt > OR_FP8ROW || d_out < 1 || d_in < 1) return -1;
  for (int64_t r = 0; r < d_out; ++r)
    for (int64_t k = 0; k < d_in; ++k)
      W[r * d_in + k] = weight(fmt, d_in, codes, scales, tensor_scale, r, k);
  return 0;
}

/* h[i] = SiLU(g[i]) * u[i] */
void or_silu_mul(int64_t n, const double* g, const double* u, double* h) {
  for (int64_t i = 0; i < n; ++i) h[i] = or_silu(g[i]) * u[i];
}

/* Router: per token m, the k experts with the largest logits (descending; equal
 * logits ordered by the lower expert index), and softmax weights over those k
 * logits (max subtracted first).  Selection by repeated scan, O(E*k). */
int or_topk_softmax(int M, int E, int k, const float* logits, int32_t* ids, double* w) {
  if (M < 1 || E < 1 || k < 1 || k > E) return -1;
  for (int m = 0; m < M; ++m) {
    const float* l = logits + (int64_t)m * E;
    int32_t* id = ids + (int64_t)m * k;
    for (int j = 0; j < k; ++j) {
      int best = -1;
      for (int e = 0; e < E; ++e) {
        int taken = 0;
        for (int q = 0; q < j; ++q)
          if (id[q] == e) taken = 1;
        if (taken) continue;
        if (best < 0 || (double)l[e] > (double)l[best]) best = e;
      }
      id[j] = best;
    }
    double mx = (double)l[id[0]], z = 0.0;
    for (int j = 1; j < k; ++j)
      if ((double)l[id[j]] > mx) mx = (double)l[id[j]];
    for (int j = 0; j < k; ++j) z += exp((double)l[id[j]] - mx);
    for (int j = 0; j < k; ++j) w[(int64_t)m * k + j] = exp((double)l[id[j]] - mx) / z;
  }
  return 0;
}
