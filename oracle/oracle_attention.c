/*
 * oracle_attention.c -- CPU reference for the fused attention forward pass.
 * TEST INFRASTRUCTURE ONLY: the tests, the smoke check and the benchmark's
 * CPU-baseline leg are its only users.  It shares no code, header or table
 * with the HIP library.
 *
 * What it computes is the plain definition of the operation the fused kernel
 * replaces -- the attention-shaped products of the pages' GEMM/BMM/attention
 * reference ("Triton Optimization Reference (cuTile -> Triton)", opening
 * section) chained through a row softmax:
 *     S[b,i,j] = scale * sum_d Q[b,i,d] * K[b,j,d]          (j < n_k)
 *     P[b,i,j] = exp(S[b,i,j] - max_j S[b,i,j]) / sum_j exp(S[b,i,j] - max_j S[b,i,j])
 *     O[b,i,c] = sum_j P[b,i,j] * V[b,j,c]
 * (no mask: every query sees every key).  Subtracting the row maximum changes
 * nothing mathematically; it keeps exp() in range.
 *
 * Precision: 16-bit inputs decoded exactly; scores, exponentials, sums and the
 * weighted sum of V in IEEE double, each sum in ascending index order.
 *
 * Storage is row-major: Q[b*sq + i*ldq + d], K[b*sk + j*ldk + d],
 * V[b*sv + j*ldv + c], all 0 <= d, c < head_dim.
 *
 * Built together with oracle_gemm.c; OpenMP only splits the requested rows
 * across threads.
 */
#include <math.h>
#include <stdint.h>
#include <stdlib.h>
#include <string.h>

#define OA_BF16 0
#define OA_FP16 1

static double a_dec_bf16(uint16_t h) {
  uint32_t u = (uint32_t)h << 16;
  float f;
  memcpy(&f, &u, sizeof f);
  return (double)f;
}

static double a_dec_fp16(uint16_t h) {
  int sign = h >> 15, e = (h >> 10) & 0x1f, f = h & 0x3ff;
  double v;
  if (e == 0)
    v = ldexp((double)f, -24);
  else if (e == 31)
    v = f ? NAN : INFINITY;
  else
    v = ldexp((double)(f | 0x400), e - 25);
  return sign ? -v : v;
}

static double a_dec(int type, uint16_t h) { return type == OA_FP16 ? a_dec_fp16(h) : a_dec_bf16(h); }

/*
 * rows: `count` (b, i) pairs (int64, row-major [count][2]); out: [count][head_dim].
 * Returns 0, or -1 if a requested row is outside the problem or n_k < 1.
 */
int oracle_attention(int in_type, int64_t n_q, int64_t n_k, int64_t head_dim, double scale, const uint16_t* Q,
                     int64_t ldq, int64_t sq, const uint16_t* K, int64_t ldk, int64_t sk, const uint16_t* V,
                     int64_t ldv, int64_t sv, int64_t batch, const int64_t* rows, int64_t count, double* out) {
  if (n_k < 1) return -1;
  for (int64_t r = 0; r < count; ++r)
    if (rows[2 * r] < 0 || rows[2 * r] >= batch || rows[2 * r + 1] < 0 || rows[2 * r + 1] >= n_q) return -1;
  int bad = 0;
#pragma omp parallel for schedule(dynamic, 4)
  for (int64_t r = 0; r < count; ++r) {
    double* s = (double*)malloc(sizeof(double) * (size_t)n_k);
    if (!s) {
#pragma omp atomic write
      bad = 1;
      continue;
    }
    const int64_t b = rows[2 * r], i = rows[2 * r + 1];
    const uint16_t* q = Q + b * sq + i * ldq;
    /* scores and their maximum */
    double mx = -INFINITY;
    for (int64_t j = 0; j < n_k; ++j) {
      const uint16_t* kr = K + b * sk + j * ldk;
      double acc = 0.0;
      for (int64_t d = 0; d < head_dim; ++d) acc += a_dec(in_type, q[d]) * a_dec(in_type, kr[d]);
      s[j] = scale * acc;
      if (s[j] > mx) mx = s[j];
    }
    /* unnormalised weights and their sum */
    double den = 0.0;
    for (int64_t j = 0; j < n_k; ++j) {
      s[j] = exp(s[j] - mx);
      den += s[j];
    }
    /* weighted sum of V rows, normalised */
    double* o = out + r * head_dim;
    for (int64_t c = 0; c < head_dim; ++c) {
      double acc = 0.0;
      for (int64_t j = 0; j < n_k; ++j) acc += s[j] * a_dec(in_type, V[b * sv + j * ldv + c]);
      o[c] = acc / den;
    }
    free(s);
  }
  return bad ? -1 : 0;
}
