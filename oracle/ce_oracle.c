/*
 * ce_oracle.c -- TEST INFRASTRUCTURE ONLY.
 *
 * A plain, slow, obviously correct CPU reference for row-wise softmax
 * cross-entropy and its gradient, evaluated in fp64 on the stored input
 * values.  Only the test suite, the smoke check and the bench's CPU-baseline
 * leg may load this library.  The GPU library shares no code with it: no
 * header, no helper, no table.  The only parallelism is an OpenMP loop over
 * independent rows; every row is computed by one thread in the order written.
 *
 * What it computes, with the passages it follows:
 *  - The loss of row i is  lse_i - x[i, t_i]  with  lse_i = log sum_j exp(x_ij):
 *    the problem statement of the POPCORNBENCH "Kimi-K2.6 l1_p95" reasoning
 *    trace (log_softmax, then negative log-likelihood of the target, then the
 *    mean over the batch), and the last line of loss_kernel in the Triton
 *    issue "Cross Entropy Loss performance issue" (log of the sum of exps plus
 *    the max, minus the target logit).
 *  - The max-shifted form  lse = m + log sum_j exp(x_j - m)  (same trace,
 *    "per row max, subtract, exp, sum, log").
 *  - The gradient of the reduced loss with respect to the logits,
 *    (softmax(x_i) - onehot(t_i)) * c  with c = 1/M for the mean and 1 for the
 *    sum or per-row losses: "9 Triton kernels in 9 weeks", week 7 (fused
 *    forward and backward that writes the gradient over the logits buffer),
 *    optionally times an upstream gradient per row (chain rule).
 *  - Row softmax exp(x_ij - lse_i) and log-softmax x_ij - lse_i: same page,
 *    week 1 (fused softmax), and the log_softmax step of the trace's problem
 *    statement.
 *  - Linear + cross-entropy: the logits are the lm_head projection z = H W^T
 *    of bf16 hidden states H [M, D] and weight W [V, D], and the loss is the
 *    cross-entropy above on z; gradients dH = G W and dW = G^T H with G the
 *    logits' gradient: same page, week 8 (the lm_head projection folded into
 *    the loss, chunk by chunk).  Products of two bf16 values are exact in
 *    fp64; their sums are plain fp64 sums.
 *
 * Readings taken where the pages are silent (each is listed in the design
 * notes of the repository):
 *  - A target outside [0, V) gives a NaN loss; its gradient row is
 *    softmax * c with no one-hot term.
 *  - A NaN or +inf logit gives a NaN loss and NaN gradient row.  A row that
 *    is entirely -inf has lse = -inf and a NaN loss.  A -inf target logit
 *    (with a finite max) gives +inf.
 *  - Mean divides the compensated sum of the M row losses by M; with M = 0 it
 *    is 0/0 = NaN and the sum is 0.
 *  - Gradients are rounded once, directly from fp64 to the storage type,
 *    round-to-nearest-even, keeping subnormals.
 *
 * Accuracy devices (all exact rearrangements of the definition):
 *  - the max term exp(x_j* - m) = 1 is taken out of the sum, so
 *    log sum = log1p(sum over the other terms);
 *  - loss = (m - x_t) + log1p(s'), which loses no digits when x_t = m;
 *  - the gradient at the target is expm1(-loss) * c  (= (p_t - 1) c);
 *  - sums use Neumaier's compensated summation.
 */
#include <math.h>
#include <stdint.h>
#include <stdlib.h>
#include <string.h>

enum { OR_F32 = 0, OR_F16 = 1, OR_BF16 = 2, OR_F64 = 3 /* internal: fp64 rows */ };
enum { OR_NONE = 0, OR_MEAN = 1, OR_SUM = 2 };

/* ---------------------------------------------------------------- storage */

/* IEEE binary16: 1 sign, 5 exponent (bias 15), 10 fraction bits. */
double oracle_widen_f16(uint16_t h)
{
    int sign = (h >> 15) & 1;
    int e = (h >> 10) & 31;
    int f = h & 1023;
    double v;
    if (e == 0)
        v = ldexp((double)f, -24);                 /* zero and subnormals */
    else if (e == 31)
        v = f ? NAN : INFINITY;
    else
        v = ldexp((double)(1024 + f), e - 25);     /* (1 + f/1024) 2^(e-15) */
    return sign ? -v : v;
}

/* bfloat16: the upper 16 bits of an IEEE binary32. */
double oracle_widen_bf16(uint16_t b)
{
    int sign = (b >> 15) & 1;
    int e = (b >> 7) & 255;
    int f = b & 127;
    double v;
    if (e == 0)
        v = ldexp((double)f, -133);                /* zero and subnormals */
    else if (e == 255)
        v = f ? NAN : INFINITY;
    else
        v = ldexp((double)(128 + f), e - 134);     /* (1 + f/128) 2^(e-127) */
    return sign ? -v : v;
}

/*
 * Round a double to a binary format with `mant` fraction bits, smallest
 * normal exponent `emin` and largest finite value `maxfin`, to nearest, ties
 * to even, in one step.  Returns the rounded magnitude (or +inf).
 */
static double round_binary(double a, int mant, int emin, double maxfin)
{
    int e;
    frexp(a, &e);                 /* a in [2^(e-1), 2^e) */
    int k = e - 1;
    if (k < emin)
        k = emin;                 /* subnormal spacing */
    double q = ldexp(1.0, k - mant);
    double r = nearbyint(a / q) * q;   /* a/q is exact; default mode is RNE */
    if (r > maxfin)
        return INFINITY;
    return r;
}

uint16_t oracle_round_f16(double v)
{
    if (isnan(v))
        return 0x7e00;
    uint16_t sign = signbit(v) ? 0x8000 : 0;
    double a = fabs(v);
    if (a == 0.0)
        return sign;
    double r = isinf(a) ? INFINITY : round_binary(a, 10, -14, 65504.0);
    if (isinf(r))
        return sign | 0x7c00;
    if (r < ldexp(1.0, -14))
        return sign | (uint16_t)(r / ldexp(1.0, -24));
    int e;
    frexp(r, &e);
    int k = e - 1;
    uint16_t frac = (uint16_t)(r / ldexp(1.0, k - 10) - 1024.0);
    return sign | (uint16_t)((k + 15) << 10) | frac;
}

uint16_t oracle_round_bf16(double v)
{
    if (isnan(v))
        return 0x7fc0;
    uint16_t sign = signbit(v) ? 0x8000 : 0;
    double a = fabs(v);
    if (a == 0.0)
        return sign;
    double maxfin = ldexp(255.0, 120);  /* (2 - 2^-7) 2^127 */
    double r = isinf(a) ? INFINITY : round_binary(a, 7, -126, maxfin);
    if (isinf(r))
        return sign | 0x7f80;
    if (r < ldexp(1.0, -126))
        return sign | (uint16_t)(r / ldexp(1.0, -133));
    int e;
    frexp(r, &e);
    int k = e - 1;
    uint16_t frac = (uint16_t)(r / ldexp(1.0, k - 7) - 128.0);
    return sign | (uint16_t)((k + 127) << 7) | frac;
}

float oracle_round_f32(double v)
{
    return (float)v;              /* C's conversion rounds to nearest even */
}

static double elem(const void *x, int dtype, int64_t k)
{
    switch (dtype) {
    case OR_F64:
        return ((const double *)x)[k];
    case OR_F32:
        return (double)((const float *)x)[k];
    case OR_F16:
        return oracle_widen_f16(((const uint16_t *)x)[k]);
    default:
        return oracle_widen_bf16(((const uint16_t *)x)[k]);
    }
}

/* --------------------------------------------------- compensated summation */

typedef struct {
    double sum, comp;
} nsum_t;

static void nsum_add(nsum_t *a, double v)
{
    double t = a->sum + v;
    if (fabs(a->sum) >= fabs(v))
        a->comp += (a->sum - t) + v;
    else
        a->comp += (v - t) + a->sum;
    a->sum = t;
}

static double nsum_value(const nsum_t *a) { return a->sum + a->comp; }

/* -------------------------------------------------------------- one row */

/*
 * Loss of one row, and its log-sum-exp.  x points at the row's first
 * element.
 */
static double row_loss(const void *x, int dtype, int64_t V, int64_t t,
                       double *lse_out)
{
    double m = -INFINITY;
    int64_t jstar = -1;
    int bad = 0;
    for (int64_t j = 0; j < V; ++j) {
        double v = elem(x, dtype, j);
        if (isnan(v) || v == INFINITY)
            bad = 1;
        if (v > m) {
            m = v;
            jstar = j;
        }
    }
    if (bad) {
        *lse_out = NAN;
        return NAN;
    }
    if (jstar < 0) {              /* every entry is -inf */
        *lse_out = -INFINITY;
        return NAN;
    }
    nsum_t s = {0.0, 0.0};
    for (int64_t j = 0; j < V; ++j)
        if (j != jstar)
            nsum_add(&s, exp(elem(x, dtype, j) - m));
    double l1p = log1p(nsum_value(&s));
    *lse_out = m + l1p;
    if (t < 0 || t >= V)
        return NAN;
    return (m - elem(x, dtype, t)) + l1p;
}

/* ----------------------------------------------------------- public API */

static const void *row_ptr(const void *x, int dtype, int64_t row, int64_t V)
{
    size_t s = dtype == OR_F32 ? 4 : 2;
    return (const char *)x + (size_t)row * (size_t)V * s;
}

/*
 * Per-row losses (and optionally log-sum-exps) of rows [row0, row0 + nrows)
 * of the row-major [M, V] matrix x.  loss_out[k] and lse_out[k] belong to
 * row row0 + k.  Returns 0, or -1 on bad arguments.
 */
int oracle_ce_loss_rows(const void *x, int dtype, const int64_t *targets,
                        int64_t M, int64_t V, int64_t row0, int64_t nrows,
                        double *loss_out, double *lse_out)
{
    if (!x || !targets || !loss_out || V < 1 || row0 < 0 || nrows < 0 ||
        row0 + nrows > M || dtype < OR_F32 || dtype > OR_BF16)
        return -1;
#pragma omp parallel for schedule(dynamic, 16)
    for (int64_t k = 0; k < nrows; ++k) {
        int64_t i = row0 + k;
        double lse;
        double l = row_loss(row_ptr(x, dtype, i, V), dtype, V, targets[i], &lse);
        loss_out[k] = l;
        if (lse_out)
            lse_out[k] = lse;
    }
    return 0;
}

/*
 * Reduction of n row losses: none is not handled here; mean = sum / n,
 * sum = compensated sum.  With n = 0 the sum is 0 and the mean NaN.
 */
double oracle_ce_reduce(const double *losses, int64_t n, int reduction)
{
    nsum_t s = {0.0, 0.0};
    for (int64_t i = 0; i < n; ++i)
        nsum_add(&s, losses[i]);
    double total = nsum_value(&s);
    if (reduction == OR_MEAN)
        return total / (double)n;
    return total;
}

/*
 * Full forward: the per-row losses of all M rows reduced as asked.  For
 * none, out receives M values; otherwise out[0] receives the scalar.
 * scratch must hold M doubles for mean and sum (it receives the row losses).
 */
int oracle_ce_fwd(const void *x, int dtype, const int64_t *targets, int64_t M,
                  int64_t V, int reduction, double *out, double *scratch)
{
    if (M < 0 || !out || reduction < OR_NONE || reduction > OR_SUM)
        return -1;
    double *losses = reduction == OR_NONE ? out : scratch;
    if (M > 0 && !losses)
        return -1;
    if (M > 0 && oracle_ce_loss_rows(x, dtype, targets, M, V, 0, M, losses, 0))
        return -1;
    if (reduction != OR_NONE)
        out[0] = oracle_ce_reduce(losses, M, reduction);
    return 0;
}

static void store_rounded(void *out, int out_dtype, size_t o, double v)
{
    if (out_dtype == OR_F32)
        ((float *)out)[o] = oracle_round_f32(v);
    else if (out_dtype == OR_F16)
        ((uint16_t *)out)[o] = oracle_round_f16(v);
    else
        ((uint16_t *)out)[o] = oracle_round_bf16(v);
}

/*
 * Gradient of rows [row0, row0 + nrows) with scale c (times d[i] when the
 * upstream gradients d are given, one per row of the whole matrix: by the
 * chain rule the gradient of sum_i d_i loss_i is d_i times that of loss_i):
 *   g_ij = exp(x_ij - lse_i) * c d_i      for j != t_i,
 *   g_it = expm1(-loss_i) * c d_i         (= (p_t - 1) c d_i).
 * A target outside [0, V) leaves out the one-hot term.  Results go to
 * grad64 (fp64, may be NULL) and to grad_out in out_dtype rounded once from
 * fp64 (may be NULL).  Both are indexed from row row0.
 */
int oracle_ce_grad_rows(const void *x, int dtype, const int64_t *targets,
                        int64_t M, int64_t V, int64_t row0, int64_t nrows,
                        double c, const double *d, int out_dtype,
                        void *grad_out, double *grad64)
{
    if (!x || !targets || V < 1 || row0 < 0 || nrows < 0 ||
        row0 + nrows > M || dtype < OR_F32 || dtype > OR_BF16 ||
        out_dtype < OR_F32 || out_dtype > OR_BF16)
        return -1;
#pragma omp parallel for schedule(dynamic, 4)
    for (int64_t k = 0; k < nrows; ++k) {
        int64_t i = row0 + k;
        const void *xr = row_ptr(x, dtype, i, V);
        int64_t t = targets[i];
        double ci = d ? c * d[i] : c;
        double lse;
        double loss = row_loss(xr, dtype, V, t, &lse);
        for (int64_t j = 0; j < V; ++j) {
            double g;
            if (j == t)
                g = expm1(-loss) * ci;
            else
                g = exp(elem(xr, dtype, j) - lse) * ci;
            size_t o = (size_t)k * (size_t)V + (size_t)j;
            if (grad64)
                grad64[o] = g;
            if (grad_out)
                store_rounded(grad_out, out_dtype, o, g);
        }
    }
    return 0;
}

/*
 * Row softmax (log_softmax == 0) or log-softmax of rows [row0, row0 + nrows):
 *   softmax_ij     = exp(x_ij - lse_i)
 *   log_softmax_ij = x_ij - lse_i
 * ("9 Triton kernels in 9 weeks", week 1: fused row softmax; the
 * log_softmax of the POPCORNBENCH "Kimi-K2.6 l1_p95" trace's problem
 * statement).  lse_i is the row's log-sum-exp as in row_loss.  A row that is
 * entirely -inf has lse = -inf and gives NaN everywhere.  Outputs as for the
 * gradient; lse_out (may be NULL) receives the fp64 lse of each row.
 */
int oracle_softmax_rows(const void *x, int dtype, int64_t M, int64_t V,
                        int64_t row0, int64_t nrows, int log_softmax,
                        int out_dtype, void *out, double *out64,
                        double *lse_out)
{
    if (!x || V < 1 || row0 < 0 || nrows < 0 || row0 + nrows > M ||
        dtype < OR_F32 || dtype > OR_BF16 || out_dtype < OR_F32 ||
        out_dtype > OR_BF16)
        return -1;
#pragma omp parallel for schedule(dynamic, 4)
    for (int64_t k = 0; k < nrows; ++k) {
        const void *xr = row_ptr(x, dtype, row0 + k, V);
        double lse;
        row_loss(xr, dtype, V, -1, &lse);
        if (lse_out)
            lse_out[k] = lse;
        for (int64_t j = 0; j < V; ++j) {
            double v = elem(xr, dtype, j) - lse;
            if (!log_softmax)
                v = exp(v);
            size_t o = (size_t)k * (size_t)V + (size_t)j;
            if (out64)
                out64[o] = v;
            if (out)
                store_rounded(out, out_dtype, o, v);
        }
    }
    return 0;
}

/*
 * The gradient, softmax or log-softmax of single elements, from the row's
 * log-sum-exp as oracle_ce_loss_rows returns it (every one of these outputs
 * depends only on its own logit once lse_i is known, so a sample of a very
 * long row needs one pass over the row, not one per output).  For k < n,
 * element (rows[k], cols[k]) of the [M, V] matrix x:
 *   op 0:  g = (exp(x_ij - lse_i) - [j == t_i]) * c d_i, the target term as
 *          expm1(x_it - lse_i) * c d_i (same page, week 7, and the chain rule
 *          for d as in oracle_ce_grad_rows; d may be NULL);
 *   op 1:  exp(x_ij - lse_i);   op 2:  x_ij - lse_i   (week 1, the trace).
 * lse has one entry per row of x.  Results go to out64[k] (fp64, may be
 * NULL) and out[k] in out_dtype rounded once (may be NULL).
 */
int oracle_at_elements(const void *x, int dtype, const int64_t *targets,
                       int64_t M, int64_t V, const double *lse, int64_t n,
                       const int64_t *rows, const int64_t *cols, int op,
                       double c, const double *d, int out_dtype, void *out,
                       double *out64)
{
    if (!x || !lse || !rows || !cols || n < 0 || V < 1 || op < 0 || op > 2 ||
        (op == 0 && !targets) || dtype < OR_F32 || dtype > OR_BF16 ||
        out_dtype < OR_F32 || out_dtype > OR_BF16)
        return -1;
    for (int64_t k = 0; k < n; ++k)
        if (rows[k] < 0 || rows[k] >= M || cols[k] < 0 || cols[k] >= V)
            return -1;
    for (int64_t k = 0; k < n; ++k) {
        int64_t i = rows[k], j = cols[k];
        double u = elem(row_ptr(x, dtype, i, V), dtype, j) - lse[i];
        double v;
        if (op == 0) {
            double ci = d ? c * d[i] : c;
            v = (j == targets[i] ? expm1(u) : exp(u)) * ci;
        } else {
            v = op == 1 ? exp(u) : u;
        }
        if (out64)
            out64[k] = v;
        if (out)
            store_rounded(out, out_dtype, (size_t)k, v);
    }
    return 0;
}

/*
 * Linear + cross-entropy on bf16 H [M, D] and W [V, D] (bit patterns):
 * z_i = H_i W^T in fp64, then row_loss on z_i.  out: per-row losses (none)
 * or the reduced loss in out[0]; lse_out [M] (may be NULL).  When G is not
 * NULL it receives the logits' gradient [M, V] with scale c (1/M for mean,
 * else 1); dH [M, D] = G W and dW [V, D] = G^T H (each may be NULL; both
 * need G).  Returns 0, or -1 on bad arguments or no memory.
 */
int oracle_linear_ce(const uint16_t *H, const uint16_t *W, const int64_t *targets,
                     int64_t M, int64_t D, int64_t V, int reduction,
                     double *out, double *lse_out, double *G, double *dH,
                     double *dW)
{
    if (!H || !W || !targets || !out || M < 0 || D < 1 || V < 1 ||
        reduction < OR_NONE || reduction > OR_SUM || ((dH || dW) && !G))
        return -1;
    double *losses = (double *)malloc(sizeof(double) * (size_t)(M > 0 ? M : 1));
    if (!losses)
        return -1;
    const double c = reduction == OR_MEAN ? 1.0 / (double)M : 1.0;
    int fail = 0;
#pragma omp parallel for schedule(dynamic, 1)
    for (int64_t i = 0; i < M; ++i) {
        double *z = (double *)malloc(sizeof(double) * (size_t)V);
        if (!z) {
            fail = 1;
            continue;
        }
        for (int64_t j = 0; j < V; ++j) {
            double acc = 0.0;
            for (int64_t k = 0; k < D; ++k)
                acc += oracle_widen_bf16(H[i * D + k]) * oracle_widen_bf16(W[j * D + k]);
            z[j] = acc;
        }
        const int64_t t = targets[i];
        double lse;
        const double loss = row_loss(z, OR_F64, V, t, &lse);
        losses[i] = loss;
        if (lse_out)
            lse_out[i] = lse;
        if (G)
            for (int64_t j = 0; j < V; ++j)
                G[i * V + j] = (j == t ? expm1(-loss) : exp(z[j] - lse)) * c;
        free(z);
    }
    if (fail) {
        free(losses);
        return -1;
    }
    if (reduction == OR_NONE)
        memcpy(out, losses, sizeof(double) * (size_t)M);
    else
        out[0] = oracle_ce_reduce(losses, M, reduction);
    free(losses);
    if (dH) {
#pragma omp parallel for schedule(static)
        for (int64_t i = 0; i < M; ++i)
            for (int64_t k = 0; k < D; ++k) {
                double acc = 0.0;
                for (int64_t j = 0; j < V; ++j)
                    acc += G[i * V + j] * oracle_widen_bf16(W[j * D + k]);
                dH[i * D + k] = acc;
            }
    }
    if (dW) {
#pragma omp parallel for schedule(static)
        for (int64_t j = 0; j < V; ++j)
            for (int64_t k = 0; k < D; ++k) {
                double acc = 0.0;
                for (int64_t i = 0; i < M; ++i)
                    acc += G[i * V + j] * oracle_widen_bf16(H[i * D + k]);
                dW[j * D + k] = acc;
            }
    }
    return 0;
}

/* Sets the number of OpenMP threads later parallel regions use (n >= 1). */
void oracle_set_num_threads(int n)
{
#ifdef _OPENMP
    extern void omp_set_num_threads(int);
    if (n >= 1)
        omp_set_num_threads(n);
#else
    (void)n;
#endif
}

/* Number of OpenMP threads a parallel region uses (for reporting). */
int oracle_num_threads(void)
{
    int n = 1;
#pragma omp parallel
    {
#pragma omp single
        {
#ifdef _OPENMP
            extern int omp_get_num_threads(void);
            n = omp_get_num_threads();
#endif
        }
    }
    return n;
}
