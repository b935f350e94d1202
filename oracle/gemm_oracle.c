/*
 * CPU oracle for C = A·Bᵀ — TEST INFRASTRUCTURE ONLY.
 *
 * Only the tests, the package's smoke entry and the benchmark's CPU-baseline leg may load
 * this library. The product (the HIP library) never calls it and shares no code with it.
 *
 * What it computes (the plain definition, written out):
 *   A[M,K] and B[N,K] are K-major matrices of fp16 or bf16 bit patterns with leading
 *   dimensions lda, ldb. For every output (i, j):
 *       S_ij = sum_{k=0}^{K-1} a_ik * b_jk       in float64, k ascending
 *       T_ij = sum_{k=0}^{K-1} |a_ik| * |b_jk|   (same pass; the tolerance scale)
 *       C_ij = round_to_nearest_even(S_ij) in the output type, one rounding from float64.
 *   Every product of two 16-bit floats is exact in float64 (at most 22 significant bits),
 *   so S carries only the float64 summation error (<= K * 2^-53 * T).
 *
 * Where this definition comes from: the tutorial "GEMM II — pipelining with TMA" (Forced
 * move; Takeaway) states that pipelining, TMA loads and the persistent launch change only
 * when work happens and by whom — same tiles, same layouts, same math, fp32 accumulate —
 * and its TMA-store epilogue casts the fp32 accumulator to the output type. "Async Data
 * Movement: TMA" (How TMA Writes a Swizzled Layout) states that swizzling changes the
 * physical arrangement, not the logical contents. So the method reaches exactly the GEMM
 * result up to rounding order, and the oracle is that result. The tutorials leave the cast's
 * rounding unspecified; we read it as round-to-nearest-even.
 *
 * Decoders and encoders are written from the IEEE-754 binary16 layout (1 sign, 5 exponent,
 * 10 fraction bits, bias 15) and from bf16 = the upper 16 bits of a binary32.
 */
#include <math.h>
#include <pthread.h>
#include <stdint.h>
#include <stdlib.h>
#include <string.h>

enum { ORACLE_F16 = 0, ORACLE_BF16 = 1, ORACLE_F32 = 2 };

/* ------------------------------------------------------------------ decoders */

double oracle_decode_f16(uint16_t h) {
  int sign = (h >> 15) & 1;
  int e = (h >> 10) & 0x1F;
  int f = h & 0x3FF;
  double v;
  if (e == 0) {
    v = ldexp((double)f, -24); /* subnormal: f * 2^-24 */
  } else if (e == 31) {
    v = f ? NAN : INFINITY;
  } else {
    v = ldexp((double)(1024 + f), e - 25); /* (1 + f/1024) * 2^(e-15) */
  }
  return sign ? -v : v;
}

double oracle_decode_bf16(uint16_t h) {
  uint32_t u = (uint32_t)h << 16;
  float f;
  memcpy(&f, &u, sizeof f);
  return (double)f;
}

double oracle_decode(int dtype, uint16_t h) {
  return dtype == ORACLE_F16 ? oracle_decode_f16(h) : oracle_decode_bf16(h);
}

/* ------------------------------------------------------------------ encoders */

/*
 * Round a float64 to nearest-even in a binary format with `p` significant bits, minimum
 * normal exponent `emin`, maximum exponent `emax`, exponent field of `ebits` bits, and
 * return its bit pattern (sign | biased exponent | fraction). Subnormals are produced,
 * overflow gives infinity, NaN gives the canonical quiet NaN.
 */
static uint32_t encode_generic(double x, int p, int emin, int emax, int ebits) {
  const int fbits = p - 1;
  const uint32_t sign_bit = 1u << (fbits + ebits);
  const uint32_t exp_all = (1u << ebits) - 1u;
  uint32_t sign = signbit(x) ? sign_bit : 0u;
  if (isnan(x)) return (exp_all << fbits) | (1u << (fbits - 1));
  double a = fabs(x);
  if (isinf(a)) return sign | (exp_all << fbits);
  if (a == 0.0) return sign;
  int E;
  (void)frexp(a, &E); /* a = f * 2^E, f in [0.5, 1) -> floor(log2 a) = E - 1 */
  int e = E - 1;
  if (e < emin) e = emin; /* subnormal range: fixed quantum 2^(emin - fbits) */
  double r = rint(ldexp(a, fbits - e)); /* exact scaling, then round half to even */
  /* r is the significand in units of the quantum 2^(e - fbits) */
  if (r >= ldexp(1.0, p)) { /* rounding carried into the next binade */
    r = ldexp(r, -1);
    e += 1;
  }
  if (e > emax) return sign | (exp_all << fbits);
  uint32_t sig = (uint32_t)r;
  if (sig < (1u << fbits)) return sign | sig; /* subnormal (or rounded down to zero) */
  uint32_t biased = (uint32_t)(e - emin + 1);
  return sign | (biased << fbits) | (sig - (1u << fbits));
}

uint16_t oracle_encode_f16(double x) { return (uint16_t)encode_generic(x, 11, -14, 15, 5); }
uint16_t oracle_encode_bf16(double x) { return (uint16_t)encode_generic(x, 8, -126, 127, 8); }
/* The same routine with binary32 parameters; the tests compare it with the C cast. */
uint32_t oracle_encode_f32_generic(double x) { return encode_generic(x, 24, -126, 127, 8); }

/* ulp of the output type at x: 2^(floor(log2|x|) - p + 1), floored at the subnormal quantum. */
double oracle_ulp(int dtype, double x) {
  int p, emin;
  if (dtype == ORACLE_F16) { p = 11; emin = -14; }
  else if (dtype == ORACLE_BF16) { p = 8; emin = -126; }
  else { p = 24; emin = -126; }
  double a = fabs(x);
  int e = emin;
  if (a != 0.0 && isfinite(a)) {
    int E;
    (void)frexp(a, &E);
    if (E - 1 > emin) e = E - 1;
  }
  return ldexp(1.0, e - p + 1);
}

/* ------------------------------------------------------------------ array helpers */

void oracle_decode_array(int dtype, int64_t n, const uint16_t* in, double* out) {
  for (int64_t i = 0; i < n; ++i) out[i] = oracle_decode(dtype, in[i]);
}

void oracle_encode_array(int dtype, int64_t n, const double* in, void* out) {
  for (int64_t i = 0; i < n; ++i) {
    if (dtype == ORACLE_F16) ((uint16_t*)out)[i] = oracle_encode_f16(in[i]);
    else if (dtype == ORACLE_BF16) ((uint16_t*)out)[i] = oracle_encode_bf16(in[i]);
    else ((float*)out)[i] = (float)in[i]; /* C cast: round-to-nearest-even in the default mode */
  }
}

void oracle_ulp_array(int dtype, int64_t n, const double* in, double* out) {
  for (int64_t i = 0; i < n; ++i) out[i] = oracle_ulp(dtype, in[i]);
}

static void store_out(int out_dtype, void* C, int64_t idx, double s) {
  if (out_dtype == ORACLE_F16) ((uint16_t*)C)[idx] = oracle_encode_f16(s);
  else if (out_dtype == ORACLE_BF16) ((uint16_t*)C)[idx] = oracle_encode_bf16(s);
  else ((float*)C)[idx] = (float)s;
}

/* ------------------------------------------------------------------ the triple loop */

typedef struct {
  int64_t M, N, K;
  int in_dtype, out_dtype;
  const uint16_t* A; int64_t lda;
  const double* Bd; /* B decoded once, dense [N, K] */
  void* C; int64_t ldc;
  double* S; double* T; /* optional, [M, N] dense */
  int64_t row_begin, row_end;
} gemm_job_t;

static void* gemm_rows(void* arg) {
  gemm_job_t* j = (gemm_job_t*)arg;
  double* arow = (double*)malloc(sizeof(double) * (size_t)(j->K > 0 ? j->K : 1));
  for (int64_t i = j->row_begin; i < j->row_end; ++i) {
    for (int64_t k = 0; k < j->K; ++k) arow[k] = oracle_decode(j->in_dtype, j->A[i * j->lda + k]);
    for (int64_t n = 0; n < j->N; ++n) {
      const double* brow = j->Bd + n * j->K;
      double s = 0.0, t = 0.0;
      for (int64_t k = 0; k < j->K; ++k) {
        s += arow[k] * brow[k];
        t += fabs(arow[k]) * fabs(brow[k]);
      }
      if (j->C) store_out(j->out_dtype, j->C, i * j->ldc + n, s);
      if (j->S) j->S[i * j->N + n] = s;
      if (j->T) j->T[i * j->N + n] = t;
    }
  }
  free(arow);
  return NULL;
}

/*
 * Full product. C (optional) receives the rounded output with leading dimension ldc;
 * S and T (optional) receive the float64 sums as dense [M, N]. Rows are split over
 * `threads` POSIX threads. Returns 0, -1 on invalid arguments, -2 if out of memory.
 */
int oracle_gemm(int64_t M, int64_t N, int64_t K, int in_dtype, const uint16_t* A, int64_t lda,
                const uint16_t* B, int64_t ldb, int out_dtype, void* C, int64_t ldc,
                double* S, double* T, int threads) {
  if (M < 0 || N < 0 || K < 0 || lda < K || ldb < K || (C && ldc < N)) return -1;
  if (in_dtype != ORACLE_F16 && in_dtype != ORACLE_BF16) return -1;
  if (M == 0 || N == 0) return 0;
  double* Bd = (double*)malloc(sizeof(double) * (size_t)(N * (K > 0 ? K : 1)));
  if (!Bd) return -2;
  for (int64_t n = 0; n < N; ++n)
    for (int64_t k = 0; k < K; ++k) Bd[n * K + k] = oracle_decode(in_dtype, B[n * ldb + k]);
  if (threads < 1) threads = 1;
  if (threads > M) threads = (int)M;
  pthread_t* tid = (pthread_t*)calloc((size_t)threads, sizeof(pthread_t));
  gemm_job_t* jobs = (gemm_job_t*)calloc((size_t)threads, sizeof(gemm_job_t));
  for (int t = 0; t < threads; ++t) {
    gemm_job_t j = {M, N, K, in_dtype, out_dtype, A, lda, Bd, C, ldc, S, T,
                    M * t / threads, M * (t + 1) / threads};
    jobs[t] = j;
    if (t > 0) pthread_create(&tid[t], NULL, gemm_rows, &jobs[t]);
  }
  gemm_rows(&jobs[0]);
  for (int t = 1; t < threads; ++t) pthread_join(tid[t], NULL);
  free(tid);
  free(jobs);
  free(Bd);
  return 0;
}

/*
 * Sampled outputs: for each q < nsamp, the same sums for (ii[q], jj[q]). C receives the
 * rounded value at index q (uint16 bits or float), S and T the float64 sums.
 */
int oracle_gemm_sampled(int64_t M, int64_t N, int64_t K, int in_dtype, const uint16_t* A, int64_t lda,
                        const uint16_t* B, int64_t ldb, int out_dtype, int64_t nsamp,
                        const int64_t* ii, const int64_t* jj, void* C, double* S, double* T) {
  if (M < 0 || N < 0 || K < 0 || lda < K || ldb < K) return -1;
  for (int64_t q = 0; q < nsamp; ++q) {
    int64_t i = ii[q], n = jj[q];
    if (i < 0 || i >= M || n < 0 || n >= N) return -1;
    double s = 0.0, t = 0.0;
    for (int64_t k = 0; k < K; ++k) {
      double a = oracle_decode(in_dtype, A[i * lda + k]);
      double b = oracle_decode(in_dtype, B[n * ldb + k]);
      s += a * b;
      t += fabs(a) * fabs(b);
    }
    if (C) store_out(out_dtype, C, q, s);
    if (S) S[q] = s;
    if (T) T[q] = t;
  }
  return 0;
}
