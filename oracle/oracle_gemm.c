/*
 * oracle_gemm.c -- CPU reference for the tiled GEMM/BMM.  TEST INFRASTRUCTURE
 * ONLY: the tests, the smoke check and the benchmark's CPU-baseline leg are its
 * only users.  It shares no code, header or table with the HIP library.
 *
 * What it computes is the plain definition of the product the pages tune:
 *     C[b,i,j] = sum_{k=0}^{K-1} op(A[b])[i,k] * op(B[b])[k,j]
 * (2*M*N*K flops per matrix: p2 "Optimize Triton Block Parameters", Step 1),
 * where op() is an optional transpose that is nothing but a swap of the two
 * strides used to address the stored operand (p1 "Triton Optimization
 * Reference", section 2, transpose through pointer arithmetic), and the batch
 * index only offsets each operand's base by a per-operand batch stride (p1
 * section 3, 2D grid with the batch on its own axis).  Elements past K do not
 * contribute (p1 section 1: masked loads fill them with zero).
 *
 * Precision: every 16-bit input is decoded exactly, each product is formed and
 * accumulated in IEEE double, in ascending k.  A bf16 x bf16 or fp16 x fp16
 * product is exact in double; only the running sum rounds.
 *
 * Storage is row-major.  With trans_a = 0, A is M x K at A[i*lda + k]; with
 * trans_a = 1, A is stored K x M and op(A)[i,k] = A[k*lda + i].  Likewise for B:
 * trans_b = 0 stores K x N (B[k*ldb + j]); trans_b = 1 stores N x K
 * (B[j*ldb + k]).
 *
 * Built with gcc -O2 -fopenmp -shared; OpenMP only splits the output elements
 * across threads -- the sum for one element is one sequential loop.
 */
#include <math.h>
#include <stdint.h>
#include <string.h>

#define OR_BF16 0
#define OR_FP16 1

/* bf16 is the upper half of an IEEE binary32 pattern. */
static double dec_bf16(uint16_t h) {
  uint32_t u = (uint32_t)h << 16;
  float f;
  memcpy(&f, &u, sizeof f);
  return (double)f;
}

/* IEEE binary16: 1 sign, 5 exponent (bias 15), 10 fraction bits. */
static double dec_fp16(uint16_t h) {
  int sign = h >> 15, e = (h >> 10) & 0x1f, f = h & 0x3ff;
  double v;
  if (e == 0)
    v = ldexp((double)f, -24); /* subnormal: f * 2^-14 / 2^10 */
  else if (e == 31)
    v = f ? NAN : INFINITY;
  else
    v = ldexp((double)(f | 0x400), e - 25); /* (1 + f/2^10) * 2^(e-15) */
  return sign ? -v : v;
}

static double dec(int type, uint16_t h) { return type == OR_FP16 ? dec_fp16(h) : dec_bf16(h); }

/* One output element, straight from the definition. */
static double dot_one(int type, int ta, int tb, int64_t k_len, const uint16_t* A, int64_t lda,
                      const uint16_t* B, int64_t ldb, int64_t i, int64_t j) {
  double s = 0.0;
  for (int64_t k = 0; k < k_len; ++k) {
    double a = dec(type, A[ta ? k * lda + i : i * lda + k]);
    double b = dec(type, B[tb ? j * ldb + k : k * ldb + j]);
    s += a * b;
  }
  return s;
}

/*
 * oracle_gemm: fp64 reference for C[b] = op(A[b]) op(B[b]).
 *   idx == NULL : every element; out is dense [batch][m][n].
 *   idx != NULL : n_idx (b, i, j) triples (int64, row-major [n_idx][3]);
 *                 out[t] is element t.
 * Returns 0, or -1 for an index outside the problem.
 */
int oracle_gemm(int in_type, int trans_a, int trans_b, int64_t m, int64_t n, int64_t k,
                const uint16_t* A, int64_t lda, int64_t stride_a, const uint16_t* B, int64_t ldb,
                int64_t stride_b, int64_t batch, const int64_t* idx, int64_t n_idx, double* out) {
  if (idx) {
    int bad = 0;
#pragma omp parallel for schedule(dynamic, 64) reduction(| : bad)
    for (int64_t t = 0; t < n_idx; ++t) {
      int64_t b = idx[3 * t], i = idx[3 * t + 1], j = idx[3 * t + 2];
      if (b < 0 || b >= batch || i < 0 || i >= m || j < 0 || j >= n) {
        out[t] = NAN;
        bad = 1;
        continue;
      }
      out[t] = dot_one(in_type, trans_a, trans_b, k, A + b * stride_a, lda, B + b * stride_b, ldb, i, j);
    }
    return bad ? -1 : 0;
  }
  int64_t rows = batch * m;
#pragma omp parallel for schedule(dynamic, 1)
  for (int64_t r = 0; r < rows; ++r) {
    int64_t b = r / m, i = r % m;
    for (int64_t j = 0; j < n; ++j)
      out[r * n + j] = dot_one(in_type, trans_a, trans_b, k, A + b * stride_a, lda, B + b * stride_b, ldb, i, j);
  }
  return 0;
}

/* Largest |x| over a whole decoded tensor (the tolerance scales with it). */
double oracle_max_abs(int in_type, const uint16_t* X, int64_t count) {
  double mx = 0.0;
#pragma omp parallel for reduction(max : mx)
  for (int64_t t = 0; t < count; ++t) {
    double v = fabs(dec(in_type, X[t]));
    if (v > mx) mx = v;
  }
  return mx;
}

/* Decode a tensor to double (exact). */
void oracle_decode(int in_type, const uint16_t* X, int64_t count, double* out) {
#pragma omp parallel for
  for (int64_t t = 0; t < count; ++t) out[t] = dec(in_type, X[t]);
}

/*
 * Round a double to the nearest bf16 / fp16 value, ties to even, with IEEE
 * overflow to infinity and gradual underflow.  p = significand bits including
 * the hidden one, emin = exponent of the smallest normal, bias = exponent bias.
 */
static uint16_t encode_rne(double x, int p, int emin, int emax, int bias, uint16_t qnan) {
  if (isnan(x)) return qnan;
  uint16_t sign = signbit(x) ? 0x8000 : 0;
  double ax = fabs(x);
  uint16_t inf = (uint16_t)(sign | (((1u << (15 - (p - 1))) - 1u) << (p - 1)));
  if (isinf(ax)) return inf;
  if (ax == 0.0) return sign;
  int e2;
  frexp(ax, &e2);          /* ax = f * 2^e2, f in [0.5, 1): leading bit at 2^(e2-1) */
  int lead = e2 - 1;
  int q = (lead < emin ? emin : lead) - (p - 1); /* exponent of one unit in the last place */
  double r = ldexp(ax, -q);                     /* exact: a power-of-two scaling */
  double nq = nearbyint(r);                      /* default mode: round half to even */
  double v = ldexp(nq, q);
  double maxfin = ldexp(ldexp(1.0, p) - 1.0, emax - (p - 1));
  if (v > maxfin) return inf;
  if (nq == 0.0) return sign;
  frexp(v, &e2);
  lead = e2 - 1;
  uint32_t field, mant;
  if (lead < emin) {
    field = 0;
    mant = (uint32_t)ldexp(v, -(emin - (p - 1)));
  } else {
    field = (uint32_t)(lead + bias);
    mant = (uint32_t)(ldexp(v, -(lead - (p - 1))) - ldexp(1.0, p - 1));
  }
  return (uint16_t)(sign | (field << (p - 1)) | mant);
}

/* out_type 0: bf16 (8-bit significand, exponents -126..127); 1: fp16 (11-bit, -14..15). */
void oracle_round(int out_type, const double* x, int64_t count, uint16_t* bits) {
#pragma omp parallel for
  for (int64_t t = 0; t < count; ++t)
    bits[t] = out_type == OR_FP16 ? encode_rne(x[t], 11, -14, 15, 15, 0x7e00)
                                  : encode_rne(x[t], 8, -126, 127, 127, 0x7fc0);
}
