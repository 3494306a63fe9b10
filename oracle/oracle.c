/*
 * oracle.c -- plain CPU reference ("the oracle") for the batch-invariant
 * W8A16 decode projection, the fixed-block fp32 target logprob and the
 * column-local glue of one decode layer.
 *
 * TEST INFRASTRUCTURE ONLY.  It is loaded by the test suite, by the smoke
 * check and by the benchmark's CPU-baseline leg, and by nothing else.  It
 * shares no code, header, table or constant with the GPU library; the two
 * meet only through the seeded inputs of the synth package.
 *
 * What is computed, and from where (the pages):
 *  - ninfer issue "t-dependent kernel dispatch" (GitHub issue 80), table
 *    "Where t selects arithmetic", row "ops::linear W8G32": int8 weights with
 *    one scale per 32 consecutive K elements and 16-bit activations; the
 *    "Proposal" section: each output column depends on its own activation
 *    column only, so y[:, j] = dequant(W) x[:, j]
 *    is a per-column result.  The oracle is that definition written out:
 *    every term q * s * x is exact in fp64 (7 + 11 + 8 significant bits) and
 *    the terms are summed in fp64 in ascending k.
 *  - tokenspeed "Numerics envelopes": the alignment.trainer table row for
 *    "--logprob-order blockwise" (row max, shift, target gather, sum_exp over
 *    fixed-width vocabulary blocks, each block in its own fixed tree, an fp32
 *    left fold across blocks, result -(log(sum_exp) - target)), the
 *    "Logprobs" section (bf16 logits widened exactly to fp32; the trainer's
 *    negative cross-entropy gives -0.0 for a certain token) and the
 *    block_sumexp leaf contract paragraph (input already shifted by the row
 *    max, block partials returned in vocabulary order, folded left to right).
 *    That is an algorithm, so the oracle takes its steps in that order.
 *
 * Readings where the pages are silent (each one is listed in the design
 * notes): the in-block tree is the balanced pairwise tree in index order;
 * a vocabulary that is not a whole number of blocks is padded with virtual
 * -inf logits (exp gives +0); EXP32(x) and LOG32(x) are the correctly
 * rounded fp32 values of e^x and ln x, taken here from long-double libm and
 * rounded once to fp32; a NaN anywhere in a row or a target outside [0, V)
 * gives NaN.
 *
 * Build: gcc -O2 -fopenmp -ffp-contract=off -fno-fast-math -fPIC -shared.
 */
#include <math.h>
#include <omp.h>
#include <stdint.h>
#include <stdlib.h>
#include <string.h>

/* ---------------------------------------------------------------- formats */

/* bfloat16: the upper 16 bits of an IEEE binary32. */
static float bf16_as_float(uint16_t b) {
    uint32_t u = (uint32_t)b << 16;
    float f;
    memcpy(&f, &u, sizeof f);
    return f;
}

/* IEEE binary16 decoded from its fields: subnormals are m * 2^-24, normals
 * (1024 + m) * 2^(e - 25). */
static double f16_as_double(uint16_t h) {
    int sign = h >> 15, e = (h >> 10) & 0x1f, m = h & 0x3ff;
    double v;
    if (e == 0)
        v = ldexp((double)m, -24);
    else if (e == 31)
        v = m ? NAN : INFINITY;
    else
        v = ldexp((double)(m | 0x400), e - 25);
    return sign ? -v : v;
}

double oracle_bf16_value(uint16_t b) { return (double)bf16_as_float(b); }
double oracle_f16_value(uint16_t h) { return f16_as_double(h); }

/* Round a double to the nearest bfloat16 (ties to even), directly from the
 * double: scale onto the bf16 grid of the value's binade (8 significant
 * bits; the subnormal grid 2^-133 below 2^-126), round to an integer with
 * the default nearest-even mode, scale back.  Overflow past the largest
 * finite bf16 gives infinity. */
uint16_t oracle_bf16_round(double v) {
    if (isnan(v)) return 0x7FC0;
    uint16_t sign = signbit(v) ? 0x8000 : 0;
    double a = fabs(v);
    if (isinf(a)) return sign | 0x7F80;
    if (a == 0.0) return sign;
    int e;
    frexp(a, &e);            /* a = f * 2^e with f in [0.5, 1) */
    int ex = e - 1;          /* floor(log2 a) */
    if (ex < -126) ex = -126;
    double ulp = ldexp(1.0, ex - 7);
    double r = nearbyint(a / ulp) * ulp;
    const double bf16_max = ldexp(255.0, 120); /* (2 - 2^-7) * 2^127 */
    if (r > bf16_max) return sign | 0x7F80;
    float f = (float)r;      /* exact: r has at most 8 significant bits */
    uint32_t u;
    memcpy(&u, &f, sizeof u);
    return sign | (uint16_t)(u >> 16);
}

int oracle_max_threads(void) { return omp_get_max_threads(); }

/* ------------------------------------------------------------ W8G32 GEMM */

/* y[j * nrows + i] = sum_{k < K} q[n, k] * s[n, k / 32] * x[j, k],  n = rows[i]
 * (n = i when rows is NULL), for every column j < t.
 *   q : int8  [N, K] row-major (N output rows)
 *   s : fp16  [N, K/32] row-major, one scale per row and 32 consecutive k
 *   x : bf16  [t, ldx] row-major (column j of the activations is row j here)
 * Each row's weights are dequantised once into fp64 (exact), then each column
 * is a plain fp64 dot product in ascending k.
 * When mass != NULL it also receives the absolute sum of the same terms,
 * mass[j * nrows + i] = sum_k |q[n, k] * s[n, k / 32] * x[j, k]|: the scale
 * below which an fp32 accumulation of these terms cannot resolve the result
 * (one fp32 ulp of a partial sum of that size). */
void oracle_w8_linear(const int8_t *q, const uint16_t *s, const uint16_t *x,
                      int64_t N, int64_t K, int64_t t, int64_t ldx,
                      const int64_t *rows, int64_t nrows, double *y, double *mass) {
    const int64_t G = K / 32;
    (void)N;
#pragma omp parallel
    {
        double *w = (double *)malloc((size_t)K * sizeof(double));
#pragma omp for schedule(dynamic, 8)
        for (int64_t i = 0; i < nrows; ++i) {
            const int64_t n = rows ? rows[i] : i;
            const int8_t *qr = q + n * K;
            const uint16_t *sr = s + n * G;
            for (int64_t k = 0; k < K; ++k)
                w[k] = (double)qr[k] * f16_as_double(sr[k / 32]);
            for (int64_t j = 0; j < t; ++j) {
                const uint16_t *xr = x + j * ldx;
                double acc = 0.0;
                for (int64_t k = 0; k < K; ++k)
                    acc += w[k] * (double)bf16_as_float(xr[k]);
                y[j * nrows + i] = acc;
                if (mass) {
                    double a = 0.0;
                    for (int64_t k = 0; k < K; ++k)
                        a += fabs(w[k] * (double)bf16_as_float(xr[k]));
                    mass[j * nrows + i] = a;
                }
            }
        }
        free(w);
    }
}

/* ------------------------------------------------------- EXP32 and LOG32 */

/* Correctly rounded fp32 exponential and logarithm: the long-double libm
 * value (64-bit significand) rounded once to fp32. */
float oracle_exp32(float x) { return (float)expl((long double)x); }
float oracle_log32(float x) { return (float)logl((long double)x); }

void oracle_exp32_array(const float *x, int64_t n, float *out) {
#pragma omp parallel for schedule(static)
    for (int64_t i = 0; i < n; ++i) out[i] = oracle_exp32(x[i]);
}

void oracle_log32_array(const float *x, int64_t n, float *out) {
#pragma omp parallel for schedule(static)
    for (int64_t i = 0; i < n; ++i) out[i] = oracle_log32(x[i]);
}

/* EXP32 of the `count` consecutive binary32 bit patterns starting at `start`. */
void oracle_exp32_bits(uint32_t start, int64_t count, float *out) {
#pragma omp parallel for schedule(static)
    for (int64_t i = 0; i < count; ++i) {
        uint32_t u = start + (uint32_t)i;
        float x;
        memcpy(&x, &u, sizeof x);
        out[i] = oracle_exp32(x);
    }
}

/* LOG32 of the `count` consecutive binary32 bit patterns starting at `start`. */
void oracle_log32_bits(uint32_t start, int64_t count, float *out) {
#pragma omp parallel for schedule(static)
    for (int64_t i = 0; i < count; ++i) {
        uint32_t u = start + (uint32_t)i;
        float x;
        memcpy(&x, &u, sizeof x);
        out[i] = oracle_log32(x);
    }
}

/* ------------------------------------------------------ block logprob */

/* Balanced pairwise tree over w (a power of two) values in index order:
 * T(i, 1) = e[i],  T(i, 2w) = T(i, w) + T(i + w, w), every add in fp32. */
static float tree_sum(const float *e, int64_t w) {
    if (w == 1) return e[0];
    float left = tree_sum(e, w / 2);
    float right = tree_sum(e + w / 2, w / 2);
    return left + right;
}

/* Fixed-order fp32 target logprob over vocabulary blocks of width `block`.
 *   logits  : bf16 [t, ldl], column j's V logits contiguous
 *   targets : int64 [t]
 *   out     : fp32 [t]
 * Per column: m = row max (fp32, exact); e_v = EXP32(l_v - m) (one fp32
 * subtraction), +0 for the virtual padding v >= V; P_b = pairwise tree over
 * block b; S = ((P_0 + P_1) + P_2) + ...; Lg = LOG32(S); s_t = l_target - m;
 * out = -(Lg - s_t).  NaN in the row or a target outside [0, V) gives NaN.
 * When partials != NULL the block partials are also written, [t, nb]. */
void oracle_block_logprob(const uint16_t *logits, const int64_t *targets,
                          int64_t block, int64_t t, int64_t V, int64_t ldl,
                          float *out, float *partials, int direct) {
    const int64_t nb = (V + block - 1) / block;
#pragma omp parallel
    {
        float *e = (float *)malloc((size_t)(nb * block) * sizeof(float));
#pragma omp for schedule(dynamic, 1)
        for (int64_t j = 0; j < t; ++j) {
            const uint16_t *l = logits + j * ldl;
            int has_nan = 0;
            float m = -INFINITY;
            for (int64_t v = 0; v < V; ++v) {
                float lv = bf16_as_float(l[v]);
                if (isnan(lv)) has_nan = 1;
                else if (lv > m) m = lv;
            }
            const int64_t tg = targets[j];
            for (int64_t v = 0; v < V; ++v) {
                float shifted = bf16_as_float(l[v]) - m;
                e[v] = oracle_exp32(shifted);
            }
            for (int64_t v = V; v < nb * block; ++v) e[v] = 0.0f;
            float S = 0.0f;
            for (int64_t b = 0; b < nb; ++b) {
                float P = tree_sum(e + b * block, block);
                if (partials) partials[j * nb + b] = P;
                S = (b == 0) ? P : S + P;
            }
            if (has_nan || tg < 0 || tg >= V) {
                out[j] = NAN;
                continue;
            }
            float Lg = oracle_log32(S);
            float st = bf16_as_float(l[tg]) - m;
            /* blockwise: -(Lg - st), -0.0 for a certain token; blockwise-direct:
             * st - Lg, +0.0 for it (tokenspeed numerics, "Logprobs") */
            if (direct) {
                out[j] = st - Lg;
            } else {
                float d = Lg - st;
                out[j] = -d;
            }
        }
        free(e);
    }
}

/* Extended-precision reference of the same quantity, for self-checks:
 * lp = (l_t - m) - ln(sum_v exp(l_v - m)) in long double. */
void oracle_logprob_ref(const uint16_t *logits, const int64_t *targets,
                        int64_t t, int64_t V, int64_t ldl, double *out) {
#pragma omp parallel for schedule(dynamic, 1)
    for (int64_t j = 0; j < t; ++j) {
        const uint16_t *l = logits + j * ldl;
        long double m = -INFINITY;
        int has_nan = 0;
        for (int64_t v = 0; v < V; ++v) {
            long double lv = bf16_as_float(l[v]);
            if (isnan(lv)) has_nan = 1;
            else if (lv > m) m = lv;
        }
        const int64_t tg = targets[j];
        if (has_nan || tg < 0 || tg >= V) {
            out[j] = NAN;
            continue;
        }
        long double sum = 0.0L;
        for (int64_t v = 0; v < V; ++v) sum += expl((long double)bf16_as_float(l[v]) - m);
        out[j] = (double)(((long double)bf16_as_float(l[tg]) - m) - logl(sum));
    }
}

/* ------------------------------------------------------------------ glue */

/* RMSNorm of each column (the H features of token j), extended precision:
 * y = x * w / sqrt(mean(x^2) + eps); w = 1 when weight is NULL. */
void oracle_rmsnorm(const uint16_t *x, const uint16_t *weight, double eps,
                    int64_t t, int64_t H, int64_t ldx, double *y) {
    for (int64_t j = 0; j < t; ++j) {
        const uint16_t *xr = x + j * ldx;
        long double ss = 0.0L;
        for (int64_t h = 0; h < H; ++h) {
            long double v = bf16_as_float(xr[h]);
            ss += v * v;
        }
        long double r = sqrtl(ss / (long double)H + (long double)eps);
        for (int64_t h = 0; h < H; ++h) {
            long double w = weight ? (long double)bf16_as_float(weight[h]) : 1.0L;
            y[j * H + h] = (double)((long double)bf16_as_float(xr[h]) * w / r);
        }
    }
}

/* SwiGLU of each column: gate = features [0, F), up = features [F, 2F);
 * y = gate / (1 + exp(-gate)) * up, extended precision. */
void oracle_swiglu(const uint16_t *gu, int64_t t, int64_t F, int64_t ldg, double *y) {
    for (int64_t j = 0; j < t; ++j) {
        const uint16_t *r = gu + j * ldg;
        for (int64_t h = 0; h < F; ++h) {
            long double g = bf16_as_float(r[h]);
            long double u = bf16_as_float(r[F + h]);
            y[j * F + h] = (double)(g / (1.0L + expl(-g)) * u);
        }
    }
}

/* Residual add of each column, exact in double. */
void oracle_add(const uint16_t *a, const uint16_t *b, int64_t t, int64_t H,
                int64_t lda, int64_t ldb, double *y) {
    for (int64_t j = 0; j < t; ++j)
        for (int64_t h = 0; h < H; ++h)
            y[j * H + h] = (double)bf16_as_float(a[j * lda + h]) + (double)bf16_as_float(b[j * ldb + h]);
}

/* Canonical greedy argmax of each column (tokenspeed numerics, "Logprobs":
 * the vocabulary-parallel argmax takes the maximum and, among equal values,
 * the lowest index; signed zeros count as equal).  Reading for NaN (the page
 * is silent): a NaN counts as larger than every number, and among NaNs the
 * lowest index wins -- what torch.argmax and numpy.argmax do.  A plain scan in
 * index order that moves only on a strictly larger value. */
void oracle_argmax(const uint16_t *logits, int64_t t, int64_t V, int64_t ldl, int64_t *out) {
#pragma omp parallel for schedule(dynamic, 1)
    for (int64_t j = 0; j < t; ++j) {
        const uint16_t *l = logits + j * ldl;
        int64_t best = 0;
        float bv = bf16_as_float(l[0]);
        for (int64_t v = 1; v < V; ++v) {
            const float lv = bf16_as_float(l[v]);
            if (isnan(bv)) break;                  /* the first NaN is the answer */
            if (isnan(lv) || lv > bv) {
                best = v;
                bv = lv;
            }
        }
        out[j] = best;
    }
}
