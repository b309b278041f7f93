/*
 * oracle.c -- plain CPU reference for the fused SwiGLU MLP GEMM.
 *
 * TEST INFRASTRUCTURE ONLY.  Nothing on the product path may include, link,
 * load or call this file: only the test suite, the smoke check and the
 * benchmark's CPU-baseline leg use it.  It shares no header, source, table or
 * helper with the HIP library; both sides receive the same bf16 bit patterns
 * from the seeded input generator and nothing else.
 *
 * Source of truth: the gist.science page "Riepilogo Tecnico: Sovrapposizione
 * delle Attivazioni a Livello di Tile per l'Inferenza Efficiente di LLM"
 * (a summary of arXiv 2607.02521), cited below as [RT].
 *
 *   [RT §Definizione del Problema]  the gated MLP output is
 *       Y = SiLU(A x W1) (.) (A x W2): two independent matrix products, then an
 *       element-wise gate (SiLU of the first product times the second).
 *   [RT §Metodologia, Kernel-2]      the fused weight W_fused has K rows and
 *       2N columns; column 2n holds W1[:,n] (Gate) and column 2n+1 holds
 *       W2[:,n] (Up); the epilogue pairs D[m,2n] with D[m,2n+1].
 *   [RT §Contributi Chiave, item 3] accuracy is judged against an FP32
 *       reference, so this oracle works in fp32 (the page fixes the precision).
 *
 * Arithmetic, element by element (this is the plain definition; loops may be
 * interchanged but every output element sees exactly this sequence):
 *     a, w1, w2 : exact fp32 decodes of the bf16 inputs (bits << 16)
 *     g = ((a[m,0]*w1[0,n]) + a[m,1]*w1[1,n]) + ... ,  k ascending, each
 *         product and each sum rounded to fp32 separately (no FMA contraction:
 *         build with -ffp-contract=off)
 *     u = the same with w2
 *     s = g / (1 + expf(-g))             SiLU with beta = 1 ("Swish")
 *     y = s * u                            fp32, returned unrounded
 * Rounding to bf16 (round-to-nearest-even) is a separate, explicit step.
 *
 * FP8 inputs (OCP E4M3 codes with per-tensor scales; the reading is stated
 * at the FP8 section below): exact decode, round-to-nearest-even saturating
 * quantisation, the k-contiguous Gate/Up pairing of the weights, and the same
 * forward on the decoded values with an exact (fp64) dot product.
 *
 * Parity pins (the tests check this file against facts that do not come from
 * it): exact brute force with correctly rounded sums on tiny shapes, SiLU
 * closed forms, the A = I special case, invariants (W1 = 0 or W2 = 0 gives 0,
 * interleaved equals separate bit for bit, permutation equivariance, scaling
 * W2 by a power of two scales Y by it) and a float64 cross-check at full size.
 */
#include <math.h>
#include <pthread.h>
#include <stdint.h>
#include <stdlib.h>
#include <string.h>

#define ORACLE_LAYOUT_SEPARATE 0
#define ORACLE_LAYOUT_INTERLEAVED 1

/* Exact decode of a bf16 bit pattern: bf16 is the upper half of an fp32. */
static float bf16_to_f32(uint16_t h) {
  uint32_t bits = (uint32_t)h << 16;
  float f;
  memcpy(&f, &bits, sizeof f);
  return f;
}

/* fp32 -> bf16, round to nearest, ties to even, on the bit pattern.
 * NaN stays NaN (quietened); infinities and overflow behave as IEEE rounding
 * says (values that round past the largest finite bf16 become infinity). */
static uint16_t f32_to_bf16_rne(float f) {
  uint32_t bits;
  memcpy(&bits, &f, sizeof bits);
  if ((bits & 0x7f800000u) == 0x7f800000u && (bits & 0x007fffffu) != 0u)
    return (uint16_t)((bits >> 16) | 0x0040u);
  uint32_t lsb = (bits >> 16) & 1u;
  bits += 0x7fffu + lsb;
  return (uint16_t)(bits >> 16);
}

/* SiLU(x) = x * sigmoid(x) = x / (1 + e^-x), in fp32.  For x << 0 the
 * exponential overflows to +inf and the quotient is -0; for x >> 0 it is x. */
static float silu_f32(float x) { return x / (1.0f + expf(-x)); }

/* Weight element w_t[k, n] for t = 0 (Gate, W1) or t = 1 (Up, W2) under either
 * storage layout.  Separate: W1, W2 are row-major [K, N].  Interleaved:
 * W_fused is row-major [K, 2N] with Gate in even and Up in odd columns. */
static float weight_at(const uint16_t* w1, const uint16_t* w2, int layout,
                       int64_t N, int64_t k, int64_t n, int t) {
  if (layout == ORACLE_LAYOUT_INTERLEAVED)
    return bf16_to_f32(w1[k * 2 * N + 2 * n + t]);
  return bf16_to_f32((t == 0 ? w1 : w2)[k * N + n]);
}

/* ------------------------------------------------------------------------ */
/* Work split over threads: each worker takes a contiguous slice of a list  */
/* of row (or column) indices.  Splitting never changes any element's sum.  */
/* ------------------------------------------------------------------------ */
typedef struct {
  const uint16_t *a, *w1, *w2;
  int layout;
  int64_t M, N, K;
  const int64_t* idx; /* rows (row mode) or columns (column mode) */
  int64_t lo, hi;     /* slice of idx this worker owns */
  float *y, *g, *u;   /* outputs; g, u may be NULL */
} job_t;

/* Row mode: output row r of y/g/u (length N) is model row idx[r].
 * For one row, g[n] for all n is accumulated together with k as the outer
 * loop; each g[n] still receives its terms in ascending k. */
static void* rows_worker(void* p) {
  job_t* j = (job_t*)p;
  const int64_t N = j->N, K = j->K;
  float* gacc = (float*)malloc(sizeof(float) * (size_t)(N > 0 ? N : 1));
  float* uacc = (float*)malloc(sizeof(float) * (size_t)(N > 0 ? N : 1));
  for (int64_t r = j->lo; r < j->hi; ++r) {
    const int64_t m = j->idx[r];
    for (int64_t n = 0; n < N; ++n) gacc[n] = 0.0f, uacc[n] = 0.0f;
    for (int64_t k = 0; k < K; ++k) {
      const float a = bf16_to_f32(j->a[m * K + k]);
      if (j->layout == ORACLE_LAYOUT_INTERLEAVED) {
        const uint16_t* wf = j->w1 + k * 2 * N; /* row k of W_fused */
        for (int64_t n = 0; n < N; ++n) {
          const float p1 = a * bf16_to_f32(wf[2 * n]);     /* Gate column */
          const float p2 = a * bf16_to_f32(wf[2 * n + 1]); /* Up column */
          gacc[n] = gacc[n] + p1;
          uacc[n] = uacc[n] + p2;
        }
      } else {
        const uint16_t* w1 = j->w1 + k * N; /* row k of W1 */
        const uint16_t* w2 = j->w2 + k * N; /* row k of W2 */
        for (int64_t n = 0; n < N; ++n) {
          const float p1 = a * bf16_to_f32(w1[n]);
          const float p2 = a * bf16_to_f32(w2[n]);
          gacc[n] = gacc[n] + p1;
          uacc[n] = uacc[n] + p2;
        }
      }
    }
    for (int64_t n = 0; n < N; ++n) {
      const float s = silu_f32(gacc[n]);
      j->y[r * N + n] = s * uacc[n];
      if (j->g) j->g[r * N + n] = gacc[n];
      if (j->u) j->u[r * N + n] = uacc[n];
    }
  }
  free(gacc), free(uacc);
  return NULL;
}

/* Column mode: output column c of y/g/u (each [M, ncols]) is model column
 * idx[c].  The column of W1 and W2 is gathered once, then every row's dot
 * product runs over k ascending -- the same sequence as row mode. */
typedef struct {
  job_t base;
  int64_t ncols;
} colsjob_t;

static void* cols_worker(void* p) {
  colsjob_t* cj = (colsjob_t*)p;
  job_t* j = &cj->base;
  const int64_t M = j->M, K = j->K, C = cj->ncols;
  float* w1col = (float*)malloc(sizeof(float) * (size_t)(K > 0 ? K : 1));
  float* w2col = (float*)malloc(sizeof(float) * (size_t)(K > 0 ? K : 1));
  for (int64_t c = j->lo; c < j->hi; ++c) {
    const int64_t n = j->idx[c];
    for (int64_t k = 0; k < K; ++k) {
      w1col[k] = weight_at(j->w1, j->w2, j->layout, j->N, k, n, 0);
      w2col[k] = weight_at(j->w1, j->w2, j->layout, j->N, k, n, 1);
    }
    for (int64_t m = 0; m < M; ++m) {
      float g = 0.0f, u = 0.0f;
      for (int64_t k = 0; k < K; ++k) {
        const float a = bf16_to_f32(j->a[m * K + k]);
        const float p1 = a * w1col[k];
        const float p2 = a * w2col[k];
        g = g + p1;
        u = u + p2;
      }
      const float s = silu_f32(g);
      j->y[m * C + c] = s * u;
      if (j->g) j->g[m * C + c] = g;
      if (j->u) j->u[m * C + c] = u;
    }
  }
  free(w1col), free(w2col);
  return NULL;
}

static int run_split(void* (*fn)(void*), void* jobs, size_t job_size, int64_t count,
                     int nthreads) {
  if (nthreads < 1) nthreads = 1;
  if (nthreads > 256) nthreads = 256;
  if ((int64_t)nthreads > count) nthreads = (int)(count > 0 ? count : 1);
  pthread_t th[256];
  int started[256] = {0};
  for (int t = 0; t < nthreads; ++t) {
    job_t* j = (job_t*)((char*)jobs + (size_t)t * job_size);
    j->lo = count * t / nthreads;
    j->hi = count * (t + 1) / nthreads;
    if (t > 0 && pthread_create(&th[t], NULL, fn, j) == 0) started[t] = 1;
  }
  /* thread 0's share (and any share whose thread could not start) runs here */
  for (int t = 0; t < nthreads; ++t) {
    if (t == 0 || !started[t]) fn((char*)jobs + (size_t)t * job_size);
  }
  for (int t = 1; t < nthreads; ++t)
    if (started[t]) pthread_join(th[t], NULL);
  return nthreads;
}

/*
 * oracle_swiglu_rows: y (and optionally g, u) for the model rows listed in
 * rows[0..nrows) (rows == NULL means all M rows in order).  Outputs are
 * row-major [nrows, N] fp32.  w2 is ignored (may be NULL) when layout is
 * interleaved, in which case w1 is W_fused [K, 2N].  Returns the number of
 * threads used, or -1 on a bad argument.
 */
int oracle_swiglu_rows(const uint16_t* a, const uint16_t* w1, const uint16_t* w2,
                       int layout, int64_t M, int64_t N, int64_t K,
                       const int64_t* rows, int64_t nrows, float* y, float* g,
                       float* u, int nthreads) {
  if (M < 0 || N < 0 || K < 0 || nrows < 0 || !y) return -1;
  if (layout != ORACLE_LAYOUT_SEPARATE && layout != ORACLE_LAYOUT_INTERLEAVED) return -1;
  if (layout == ORACLE_LAYOUT_SEPARATE && K > 0 && N > 0 && (!w1 || !w2)) return -1;
  int64_t* all = NULL;
  if (!rows) {
    nrows = M;
    all = (int64_t*)malloc(sizeof(int64_t) * (size_t)(M > 0 ? M : 1));
    for (int64_t i = 0; i < M; ++i) all[i] = i;
    rows = all;
  }
  for (int64_t i = 0; i < nrows; ++i)
    if (rows[i] < 0 || rows[i] >= M) {
      free(all);
      return -1;
    }
  job_t jobs[256];
  for (int t = 0; t < 256; ++t) {
    job_t j = {a, w1, w2, layout, M, N, K, rows, 0, 0, y, g, u};
    jobs[t] = j;
  }
  int used = run_split(rows_worker, jobs, sizeof(job_t), nrows, nthreads);
  free(all);
  return used;
}

/*
 * oracle_swiglu_cols: y (and optionally g, u) for every row and the model
 * columns listed in cols[0..ncols); outputs are row-major [M, ncols] fp32.
 * Bit-identical to oracle_swiglu_rows on shared elements.
 */
int oracle_swiglu_cols(const uint16_t* a, const uint16_t* w1, const uint16_t* w2,
                       int layout, int64_t M, int64_t N, int64_t K,
                       const int64_t* cols, int64_t ncols, float* y, float* g,
                       float* u, int nthreads) {
  if (M < 0 || N < 0 || K < 0 || ncols < 0 || !y || !cols) return -1;
  if (layout != ORACLE_LAYOUT_SEPARATE && layout != ORACLE_LAYOUT_INTERLEAVED) return -1;
  if (layout == ORACLE_LAYOUT_SEPARATE && K > 0 && N > 0 && (!w1 || !w2)) return -1;
  for (int64_t i = 0; i < ncols; ++i)
    if (cols[i] < 0 || cols[i] >= N) return -1;
  colsjob_t jobs[256];
  for (int t = 0; t < 256; ++t) {
    job_t j = {a, w1, w2, layout, M, N, K, cols, 0, 0, y, g, u};
    jobs[t].base = j;
    jobs[t].ncols = ncols;
  }
  return run_split(cols_worker, jobs, sizeof(colsjob_t), ncols, nthreads);
}

/* Element-wise SiLU in fp32 (the same function the row/column paths use). */
void oracle_silu(const float* x, float* out, int64_t n) {
  for (int64_t i = 0; i < n; ++i) out[i] = silu_f32(x[i]);
}

/* Element-wise gate: y = SiLU(g) * u in fp32.  With g, u taken from bf16
 * tensors this is what an unfused pipeline computes after materialising
 * Gate and Up [RT §Definizione del Problema: the standard implementation
 * writes both intermediates to HBM before the activation]. */
void oracle_gate(const float* g, const float* u, float* y, int64_t n) {
  for (int64_t i = 0; i < n; ++i) y[i] = silu_f32(g[i]) * u[i];
}

/* fp32 -> bf16 bit patterns, round to nearest even. */
void oracle_round_bf16(const float* x, uint16_t* out, int64_t n) {
  for (int64_t i = 0; i < n; ++i) out[i] = f32_to_bf16_rne(x[i]);
}

/* bf16 bit patterns -> fp32 (exact). */
void oracle_decode_bf16(const uint16_t* x, float* out, int64_t n) {
  for (int64_t i = 0; i < n; ++i) out[i] = bf16_to_f32(x[i]);
}

/* W_fused[k, 2n] = W1[k, n], W_fused[k, 2n+1] = W2[k, n]  [RT §Metodologia,
 * Kernel-2]: a bit copy, no arithmetic. */
void oracle_pack_interleaved(const uint16_t* w1, const uint16_t* w2, uint16_t* wf,
                             int64_t K, int64_t N) {
  for (int64_t k = 0; k < K; ++k)
    for (int64_t n = 0; n < N; ++n) {
      wf[k * 2 * N + 2 * n] = w1[k * N + n];
      wf[k * 2 * N + 2 * n + 1] = w2[k * N + n];
    }
}

/* ======================================================================== */
/* FP8 inputs                                                                */
/* ======================================================================== */
/*
 * [RT §Definizione del Problema] names FP8 quantisation as the step that makes
 * the memory-bound activation a larger share of the MLP; the page "Ottimizzazione
 * delle GEMM: la chiave per l'efficienza dei Large Language Models"
 * (§Impatto sui deployment on-premise e la sovranita dei dati) reports GEMM
 * benchmarks on MXFP8.  Neither page fixes an encoding or a scaling scheme.
 * Reading taken here: the OCP 8-bit floating-point format E4M3 (1 sign bit,
 * 4 exponent bits with bias 7, 3 mantissa bits; no infinities; S.1111.111 is
 * NaN; largest finite 448), with one fp32 scale per tensor, so that a stored
 * code q stands for the real value scale * decode(q).
 *
 * The fp8 forward is then the same definition as the bf16 one, on those real
 * values:   g = s_a s_w1 sum_k decode(a[m,k]) decode(w1[k,n]),   u likewise,
 *           y = SiLU(g) * u.
 * Every decoded product is an integer multiple of 2^-18 of magnitude at most
 * 448^2 < 2^18, so for K <= 2^17 every partial sum is a multiple of 2^-18
 * below 2^35 and an fp64 accumulator holds the dot product exactly, in any
 * order.  g and u are that exact value times s_a s_w (fp64), rounded to fp32;
 * SiLU and the product are the fp32 steps of the bf16 path above.
 */

/* Real value of an E4M3 code, from the format's definition. */
static double e4m3_value(uint8_t b) {
  const int s = b >> 7, e = (b >> 3) & 15, m = b & 7;
  double v;
  if (e == 15 && m == 7) return NAN;
  if (e == 0)
    v = ldexp((double)m, -9);      /* subnormal: (m / 8) * 2^(1 - 7) */
  else
    v = ldexp(8.0 + m, e - 10);    /* normal: (1 + m / 8) * 2^(e - 7) */
  return s ? -v : v;
}

/* fp32 -> E4M3, round to nearest with ties to even, saturating: magnitudes at
 * or above 448 (and infinities) become +-448, NaN becomes S.1111.111.  The
 * sign of zero and of values that round to zero is kept. */
static uint8_t e4m3_from_f32(float x) {
  const uint8_t sign = signbit(x) ? 0x80 : 0x00;
  if (isnan(x)) return sign | 0x7F;
  const double a = fabs((double)x);
  if (a >= 448.0) return sign | 0x7E;
  int code;
  if (a < ldexp(1.0, -6)) {
    /* below the smallest normal the codes are the multiples of 2^-9; the
     * rounded count 8 is the code of 2^-6 itself */
    code = (int)nearbyint(a * 512.0);
  } else {
    int e2;
    (void)frexp(a, &e2);          /* a in [2^(e2-1), 2^e2) */
    const int e = e2 - 1;
    const int q = (int)nearbyint(ldexp(a, 3 - e));  /* 8 .. 16 eighths of 2^e */
    code = ((e + 7) << 3) + (q - 8);                 /* q = 16 carries into e + 1 */
  }
  if (code > 0x7E) code = 0x7E;
  return (uint8_t)(sign | code);
}

void oracle_decode_e4m3(const uint8_t* x, double* out, int64_t n) {
  for (int64_t i = 0; i < n; ++i) out[i] = e4m3_value(x[i]);
}

/* q[i] = E4M3(fp32(x[i] * inv_scale)) for fp32 x: the product is rounded to
 * fp32 first, then to E4M3 as above. */
void oracle_quantize_e4m3(const float* x, float inv_scale, uint8_t* out, int64_t n) {
  for (int64_t i = 0; i < n; ++i) {
    const float v = x[i] * inv_scale;
    out[i] = e4m3_from_f32(v);
  }
}

/* W8[2n, k] = W1[k, n], W8[2n+1, k] = W2[k, n]: the Kernel-2 pairing of Gate
 * and Up columns [RT §Metodologia, Kernel-2], stored with k contiguous (each
 * W_fused column becomes a row).  A bit copy. */
void oracle_pack_fp8_kmajor(const uint8_t* w1, const uint8_t* w2, uint8_t* w8, int64_t K,
                            int64_t N) {
  for (int64_t n = 0; n < N; ++n)
    for (int64_t k = 0; k < K; ++k) {
      w8[(2 * n) * K + k] = w1[k * N + n];
      w8[(2 * n + 1) * K + k] = w2[k * N + n];
    }
}

typedef struct {
  const uint8_t *a, *w1, *w2; /* A [M, K]; W1, W2 [K, N], E4M3 codes */
  int64_t M, N, K;
  double sg, su;              /* s_a * s_w1, s_a * s_w2 */
  const int64_t* idx;
  int64_t lo, hi;
  float *y, *g, *u;
} job8_t;

static void* rows8_worker(void* p) {
  job8_t* j = (job8_t*)p;
  const int64_t N = j->N, K = j->K;
  double lut[256];
  for (int c = 0; c < 256; ++c) lut[c] = e4m3_value((uint8_t)c);
  double* gacc = (double*)malloc(sizeof(double) * (size_t)(N > 0 ? N : 1));
  double* uacc = (double*)malloc(sizeof(double) * (size_t)(N > 0 ? N : 1));
  for (int64_t r = j->lo; r < j->hi; ++r) {
    const int64_t m = j->idx[r];
    for (int64_t n = 0; n < N; ++n) gacc[n] = 0.0, uacc[n] = 0.0;
    for (int64_t k = 0; k < K; ++k) {
      const double a = lut[j->a[m * K + k]];
      const uint8_t* w1 = j->w1 + k * N;
      const uint8_t* w2 = j->w2 + k * N;
      for (int64_t n = 0; n < N; ++n) {
        gacc[n] += a * lut[w1[n]];
        uacc[n] += a * lut[w2[n]];
      }
    }
    for (int64_t n = 0; n < N; ++n) {
      const float g = (float)(gacc[n] * j->sg);
      const float u = (float)(uacc[n] * j->su);
      j->y[r * N + n] = silu_f32(g) * u;
      if (j->g) j->g[r * N + n] = g;
      if (j->u) j->u[r * N + n] = u;
    }
  }
  free(gacc), free(uacc);
  return NULL;
}

/*
 * oracle_swiglu_fp8_rows: fp32 y (and optionally g, u) of the FP8 forward for
 * the model rows listed in rows[0..nrows) (NULL: all rows).  a: E4M3 [M, K];
 * w1, w2: E4M3 [K, N] row-major; scales as described above.  Returns the
 * number of threads used, or -1 on a bad argument.
 */
int oracle_swiglu_fp8_rows(const uint8_t* a, const uint8_t* w1, const uint8_t* w2,
                           int64_t M, int64_t N, int64_t K, float s_a, float s_w1,
                           float s_w2, const int64_t* rows, int64_t nrows, float* y,
                           float* g, float* u, int nthreads) {
  if (M < 0 || N < 0 || K < 0 || nrows < 0 || !y) return -1;
  if (K > 0 && N > 0 && (!a || !w1 || !w2)) return -1;
  int64_t* all = NULL;
  if (!rows) {
    nrows = M;
    all = (int64_t*)malloc(sizeof(int64_t) * (size_t)(M > 0 ? M : 1));
    for (int64_t i = 0; i < M; ++i) all[i] = i;
    rows = all;
  }
  for (int64_t i = 0; i < nrows; ++i)
    if (rows[i] < 0 || rows[i] >= M) {
      free(all);
      return -1;
    }
  job8_t jobs[256];
  for (int t = 0; t < 256; ++t) {
    job8_t j = {a, w1, w2, M, N, K, (double)s_a * (double)s_w1, (double)s_a * (double)s_w2,
                rows, 0, 0, y, g, u};
    jobs[t] = j;
  }
  /* run_split fills lo/hi through the job_t prefix; job8_t keeps its own
   * fields, so split here */
  if (nthreads < 1) nthreads = 1;
  if (nthreads > 256) nthreads = 256;
  if ((int64_t)nthreads > nrows) nthreads = (int)(nrows > 0 ? nrows : 1);
  pthread_t th[256];
  int started[256] = {0};
  for (int t = 0; t < nthreads; ++t) {
    jobs[t].lo = nrows * t / nthreads;
    jobs[t].hi = nrows * (t + 1) / nthreads;
    if (t > 0 && pthread_create(&th[t], NULL, rows8_worker, &jobs[t]) == 0) started[t] = 1;
  }
  for (int t = 0; t < nthreads; ++t)
    if (t == 0 || !started[t]) rows8_worker(&jobs[t]);
  for (int t = 1; t < nthreads; ++t)
    if (started[t]) pthread_join(th[t], NULL);
  free(all);
  return nthreads;
}

/* ======================================================================== */
/* MXFP8 inputs (OCP Microscaling: E4M3 elements, one E8M0 scale per 32)    */
/* ======================================================================== */
/*
 * The TorchInductor/CuteDSL page (§Impatto sui deployment on-premise) reports
 * MXFP8 GEMMs.  Reading taken here: the OCP Microscaling (MX) format with E4M3
 * elements: each block of 32 consecutive elements along the reduction
 * dimension K shares one E8M0 scale byte e, which stands for 2^(e - 127)
 * (e = 255 is NaN), so element k of a row stands for 2^(e(k/32) - 127) *
 * value(q[k]).  Scales are stored row-major with a row stride of ks bytes
 * (ks >= K/32; bytes past K/32 are ignored).
 *
 * Quantisation of a block V_0..V_31 (the MX conversion rule): the shared
 * exponent is floor(log2(max |V_i|)) - 8 (8 = the exponent of E4M3's largest
 * normal, 448 = 1.75 * 2^8), clamped to [-127, 127]; an all-zero block (or one
 * of NaNs only) takes -127; each element is V_i / 2^shared rounded to E4M3 as
 * above (nearest even, saturating at 448; NaN stays NaN).  NaN elements do not
 * take part in the maximum; an infinity counts as 2^128 (shared exponent 120).
 */

static double e8m0_value(uint8_t e) { return e == 255 ? NAN : ldexp(1.0, (int)e - 127); }

/* Quantise rows of K fp32 values (row-major [rows, K], K % 32 == 0) to E4M3
 * codes q [rows, K] and E8M0 scales s [rows, ks]. */
void oracle_quantize_mx(const float* x, int64_t rows, int64_t K, int64_t ks, uint8_t* q,
                        uint8_t* s) {
  for (int64_t r = 0; r < rows; ++r) {
    for (int64_t b = 0; b < ks; ++b) s[r * ks + b] = 0;
    for (int64_t b = 0; b < K / 32; ++b) {
      const float* v = x + r * K + 32 * b;
      double amax = 0.0;
      for (int i = 0; i < 32; ++i)
        if (!isnan(v[i]) && fabs((double)v[i]) > amax) amax = fabs((double)v[i]);
      int shared = -127;
      if (isinf(amax)) {
        shared = 128 - 8; /* an infinity counts as 2^128 */
      } else if (amax > 0.0) {
        int e2;
        (void)frexp(amax, &e2); /* amax in [2^(e2-1), 2^e2): floor(log2 amax) = e2 - 1 */
        shared = (e2 - 1) - 8;
        if (shared < -127) shared = -127;
        if (shared > 127) shared = 127;
      }
      s[r * ks + b] = (uint8_t)(shared + 127);
      for (int i = 0; i < 32; ++i) {
        const double scaled = ldexp((double)v[i], -shared); /* exact: a power of two */
        q[r * K + 32 * b + i] = e4m3_from_f32((float)scaled);
      }
    }
  }
}

/* Real values of MX rows: out [rows, K] = 2^(s - 127) * value(q), fp64. */
void oracle_decode_mx(const uint8_t* q, const uint8_t* s, int64_t rows, int64_t K, int64_t ks,
                      double* out) {
  for (int64_t r = 0; r < rows; ++r)
    for (int64_t k = 0; k < K; ++k)
      out[r * K + k] = e8m0_value(s[r * ks + k / 32]) * e4m3_value(q[r * K + k]);
}

/* Fragment-ordered W_fused (the library's PACKED storage of the Kernel-2
 * matrix, [RT §Metodologia, Kernel-2]): every element W_fused[k][j] (Gate
 * W1[k][j/2] for even j, Up W2[k][j/2] for odd j) is placed at
 *   ((s*T + t)*8 + c)*512 + (16*g + l)*8 + e
 * with s = j / 128, l = (j % 128) / 8, c = j % 8, t = k / 32, g = (k % 32) / 8,
 * e = k % 8 and T = ceil(K / 32); every other position of the
 * ceil(2N / 128) * T * 4096 values is 0.  A bit copy. */
void oracle_pack_fragments(const uint16_t* w1, const uint16_t* w2, uint16_t* p, int64_t K,
                           int64_t N) {
  const int64_t S = (2 * N + 127) / 128, T = (K + 31) / 32;
  memset(p, 0, sizeof(uint16_t) * (size_t)(S * T * 4096));
  for (int64_t k = 0; k < K; ++k)
    for (int64_t j = 0; j < 2 * N; ++j) {
      const uint16_t v = (j % 2 == 0) ? w1[k * N + j / 2] : w2[k * N + j / 2];
      const int64_t s = j / 128, l = (j % 128) / 8, c = j % 8;
      const int64_t t = k / 32, g = (k % 32) / 8, e = k % 8;
      p[((s * T + t) * 8 + c) * 512 + (16 * g + l) * 8 + e] = v;
    }
}

/* Fragment-ordered W8 (the library's storage of the FP8 k-major pairing for
 * its streaming kernel): every byte W8[r][k] of W8 [R, K] is placed at
 *   ((rb*T + t)*2 + h)*1024 + (16*g + i)*16 + e
 * with rb = r / 16, i = r % 16, t = k / 128, h = (k % 128) / 64,
 * g = (k % 64) / 16, e = k % 16 and T = ceil(K / 128); every other position of
 * the ceil(R / 16) * T * 2048 bytes is 0.  A byte copy. */
void oracle_pack_fp8_fragments(const uint8_t* w8, uint8_t* p, int64_t R, int64_t K) {
  const int64_t RB = (R + 15) / 16, T = (K + 127) / 128;
  memset(p, 0, (size_t)(RB * T * 2048));
  for (int64_t r = 0; r < R; ++r)
    for (int64_t k = 0; k < K; ++k) {
      const int64_t rb = r / 16, i = r % 16;
      const int64_t t = k / 128, h = (k % 128) / 64, g = (k % 64) / 16, e = k % 16;
      p[((rb * T + t) * 2 + h) * 1024 + (16 * g + i) * 16 + e] = w8[r * K + k];
    }
}

/* Fragment-ordered W8 for the library's MXFP8 streaming kernel (K a multiple
 * of 64): every byte W8[r][k] of W8 [R, K] is placed at
 *   ((rb*T + t)*2 + v)*1024 + (i + 32*h)*16 + e
 * with rb = r / 32, i = r % 32, t = k / 64, v = (k % 64) / 32,
 * h = (k % 32) / 16, e = k % 16 and T = K / 64; every other position of the
 * ceil(R / 32) * T * 2048 bytes is 0.  A byte copy. */
void oracle_pack_mx_fragments(const uint8_t* w8, uint8_t* p, int64_t R, int64_t K) {
  const int64_t RB = (R + 31) / 32, T = K / 64;
  memset(p, 0, (size_t)(RB * T * 2048));
  for (int64_t r = 0; r < R; ++r)
    for (int64_t k = 0; k < T * 64; ++k) {
      const int64_t rb = r / 32, i = r % 32;
      const int64_t t = k / 64, v = (k % 64) / 32, h = (k % 32) / 16, e = k % 16;
      p[((rb * T + t) * 2 + v) * 1024 + (i + 32 * h) * 16 + e] = w8[r * K + k];
    }
}

/* bf16 W1, W2 [K, N] -> Wt [2N, K] bf16: row 2n = W1[:, n], row 2n+1 = W2[:, n]
 * (the Kernel-2 pairing with k contiguous), a bit copy. */
void oracle_pack_kmajor_bf16(const uint16_t* w1, const uint16_t* w2, uint16_t* wt, int64_t K,
                             int64_t N) {
  for (int64_t n = 0; n < N; ++n)
    for (int64_t k = 0; k < K; ++k) {
      wt[(2 * n) * K + k] = w1[k * N + n];
      wt[(2 * n + 1) * K + k] = w2[k * N + n];
    }
}

typedef struct {
  const uint8_t *a, *sa, *w, *sw; /* A [M,K] + SA [M,ks]; W8 [2N,K] + SW [2N,ks] */
  int64_t M, N, K, ks;
  const int64_t* idx;
  int64_t lo, hi;
  float *y, *g, *u;
} jobmx_t;

/* One output row: g[n] = sum_k a(m,k) w(2n,k), u[n] likewise with row 2n+1,
 * in fp64 over the decoded values (k ascending), then fp32 as in the bf16 path. */
static void* rowsmx_worker(void* p) {
  jobmx_t* j = (jobmx_t*)p;
  const int64_t N = j->N, K = j->K, ks = j->ks;
  double lut[256], slut[256];
  for (int c = 0; c < 256; ++c) lut[c] = e4m3_value((uint8_t)c), slut[c] = e8m0_value((uint8_t)c);
  double* arow = (double*)malloc(sizeof(double) * (size_t)(K > 0 ? K : 1));
  for (int64_t r = j->lo; r < j->hi; ++r) {
    const int64_t m = j->idx[r];
    for (int64_t k = 0; k < K; ++k)
      arow[k] = slut[j->sa[m * ks + k / 32]] * lut[j->a[m * K + k]];
    for (int64_t n = 0; n < N; ++n) {
      double gs = 0.0, us = 0.0;
      const uint8_t* wg = j->w + (2 * n) * K;
      const uint8_t* wu = j->w + (2 * n + 1) * K;
      const uint8_t* sg = j->sw + (2 * n) * ks;
      const uint8_t* su = j->sw + (2 * n + 1) * ks;
      for (int64_t k = 0; k < K; ++k) {
        gs += arow[k] * (slut[sg[k / 32]] * lut[wg[k]]);
        us += arow[k] * (slut[su[k / 32]] * lut[wu[k]]);
      }
      const float g = (float)gs, u = (float)us;
      j->y[r * N + n] = silu_f32(g) * u;
      if (j->g) j->g[r * N + n] = g;
      if (j->u) j->u[r * N + n] = u;
    }
  }
  free(arow);
  return NULL;
}

/*
 * oracle_swiglu_mx_rows: fp32 y (and optionally g, u) of the MXFP8 forward for
 * the listed rows (NULL: all).  a [M, K] + sa [M, ks]; w [2N, K] + sw [2N, ks]
 * (row 2n Gate column n, row 2n+1 Up column n).  Returns threads used or -1.
 */
int oracle_swiglu_mx_rows(const uint8_t* a, const uint8_t* sa, const uint8_t* w,
                          const uint8_t* sw, int64_t M, int64_t N, int64_t K, int64_t ks,
                          const int64_t* rows, int64_t nrows, float* y, float* g, float* u,
                          int nthreads) {
  if (M < 0 || N < 0 || K < 0 || nrows < 0 || !y || K % 32 != 0 || ks < K / 32) return -1;
  if (K > 0 && N > 0 && (!a || !sa || !w || !sw)) return -1;
  int64_t* all = NULL;
  if (!rows) {
    nrows = M;
    all = (int64_t*)malloc(sizeof(int64_t) * (size_t)(M > 0 ? M : 1));
    for (int64_t i = 0; i < M; ++i) all[i] = i;
    rows = all;
  }
  for (int64_t i = 0; i < nrows; ++i)
    if (rows[i] < 0 || rows[i] >= M) {
      free(all);
      return -1;
    }
  jobmx_t jobs[256];
  for (int t = 0; t < 256; ++t) {
    jobmx_t jb = {a, sa, w, sw, M, N, K, ks, rows, 0, 0, y, g, u};
    jobs[t] = jb;
  }
  if (nthreads < 1) nthreads = 1;
  if (nthreads > 256) nthreads = 256;
  if ((int64_t)nthreads > nrows) nthreads = (int)(nrows > 0 ? nrows : 1);
  pthread_t th[256];
  int started[256] = {0};
  for (int t = 0; t < nthreads; ++t) {
    jobs[t].lo = nrows * t / nthreads;
    jobs[t].hi = nrows * (t + 1) / nthreads;
    if (t > 0 && pthread_create(&th[t], NULL, rowsmx_worker, &jobs[t]) == 0) started[t] = 1;
  }
  for (int t = 0; t < nthreads; ++t)
    if (t == 0 || !started[t]) rowsmx_worker(&jobs[t]);
  for (int t = 1; t < nthreads; ++t)
    if (started[t]) pthread_join(th[t], NULL);
  free(all);
  return nthreads;
}
