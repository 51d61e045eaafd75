/*
 * CPU ORACLE of one data-parallel rank's sharded optimizer step.
 * TEST INFRASTRUCTURE ONLY: the tests, the smoke check and the benchmark's
 * CPU-baseline leg load it.  The GPU library never links, loads or calls it,
 * and it shares no code, header or table with that library.
 *
 * What it computes, and where the pages define it:
 *
 *  - Shard ownership.  The parameters are one flat vector (the tensor list
 *    concatenated in order); with N data-parallel ranks, rank r owns the
 *    contiguous segment [r*S, (r+1)*S), S = ceil(total / N), the last
 *    segment possibly shorter.  Each rank updates one segment only and
 *    the segments together cover every parameter once ("CS336 2026
 *    Lecture 8: Parallelism Basics", Slides 19-20: each rank is responsible
 *    for one segment of the parameters and keeps only that segment's Adam
 *    state; "并行训练优化、MoE扩展与系统瓶颈", 2.2.1).
 *
 *  - Reduce.  The gradient of the shard is the average of the N ranks'
 *    local gradients, g = (1/N) * sum_k g_k ("并行策略总览：六个维度各切什么、
 *    怎么通信", data-parallel section, the gradient-averaging identity;
 *    CS231n "Large-Scale Distributed Training" notes, 4.1).  Reduce-scatter
 *    delivers exactly the owner's slice of the all-reduce result (Lecture 8,
 *    Slide 8: all-reduce = reduce-scatter + all-gather).  The sum is taken
 *    in double, rank 0 first, adding ranks 1..N-1 in order, then divided
 *    by N; the reduced shard is handed to the optimizer as an fp32 tensor.
 *
 *  - AdamW.  The pages name the optimizer state (fp32 master weights, Adam
 *    first moment m and second moment v, Lecture 8 Slide 17) but never write
 *    the update.  The reading taken is decoupled-weight-decay Adam
 *    (Loshchilov & Hutter) with bias correction, eps outside the root:
 *        m' = b1 m + (1 - b1) g
 *        v' = b2 v + (1 - b2) g^2
 *        mhat = m' / (1 - b1^t),  vhat = v' / (1 - b2^t)
 *        theta' = theta (1 - lr wd) - lr mhat / (sqrt(vhat) + eps)
 *    every operation in IEEE double, each stored result rounded once to
 *    fp32 (round-to-nearest-even).
 *
 *  - Parameter write.  The bf16 parameter is the fp32 master rounded to
 *    nearest-even bf16 (mixed precision keeps 16-bit parameters beside the
 *    fp32 master, Lecture 8 Slide 17), written into the rank's slot of the
 *    full parameter buffer: the local half of the parameter all-gather
 *    (Lecture 8 Slide 20, fourth step).  NaN stays NaN (quiet bit set,
 *    sign kept); overflow rounds to infinity.
 *
 * The storage formats (bf16 parameters and gradient partials, fp32 master,
 * m, v) are the ones the pages fix in the 16-bytes-per-parameter ledger
 * (Lecture 8 Slide 17); the arithmetic precision is not fixed there, so
 * the oracle computes in double.
 *
 * Built with gcc -O2 -ffp-contract=off -fno-fast-math: no fused
 * multiply-add, IEEE double on SSE2, correctly rounded sqrt and division.
 */
#include <math.h>
#include <stdint.h>
#include <string.h>
#ifdef _OPENMP
#include <omp.h>
#endif

enum { ORACLE_BF16 = 0, ORACLE_FP32 = 1 };

/* Loops over fewer elements than this run on the calling thread (elements
 * are independent, so the split never changes a result). */
#define ORACLE_PAR_MIN 16384

typedef struct {
    double lr, beta1, beta2, eps, weight_decay;
    int64_t step; /* t >= 1: the number of this update, counted from 1 */
} oracle_hparams;

/* ---- bf16 <-> fp32 ---------------------------------------------------- */

static double bf16_value(uint16_t h)
{
    uint32_t u = (uint32_t)h << 16; /* bf16 is the high half of an fp32 */
    float f;
    memcpy(&f, &u, 4);
    return (double)f;
}

/*
 * Nearest-even rounding of an fp32 to bf16: keep the high 16 bits, then
 * look at the 16 dropped bits.  Above half an ulp: round up.  Exactly half:
 * round up only if the kept pattern is odd.  Rounding up is +1 on the
 * 16-bit pattern; a carry out of the significand moves into the exponent,
 * which is the right result (and turns the largest finite value into inf).
 */
uint16_t oracle_bf16_round(float x)
{
    uint32_t u;
    memcpy(&u, &x, 4);
    uint16_t hi = (uint16_t)(u >> 16);
    uint32_t dropped = u & 0xFFFFu;
    int is_nan = ((u & 0x7F800000u) == 0x7F800000u) && (u & 0x007FFFFFu);
    if (is_nan)
        return (uint16_t)(hi | 0x0040u);
    if (dropped > 0x8000u || (dropped == 0x8000u && (hi & 1u)))
        hi = (uint16_t)(hi + 1u);
    return hi;
}

void oracle_bf16_round_array(const float *in, int64_t n, uint16_t *out)
{
#pragma omp parallel for schedule(static) if (n > ORACLE_PAR_MIN)
    for (int64_t i = 0; i < n; ++i)
        out[i] = oracle_bf16_round(in[i]);
}

/* ---- the three steps, per element ------------------------------------- */

static double partial_at(const void *p, int gdt, int64_t i)
{
    if (gdt == ORACLE_BF16)
        return bf16_value(((const uint16_t *)p)[i]);
    return (double)((const float *)p)[i];
}

static float reduce_one(const void *const *partials, int n_ranks, int gdt, int64_t i)
{
    double s = partial_at(partials[0], gdt, i);
    for (int k = 1; k < n_ranks; ++k)
        s = s + partial_at(partials[k], gdt, i);
    return (float)(s / (double)n_ranks);
}

static void adamw_one(float g32, float *theta, float *m, float *v, const oracle_hparams *hp,
                      double bc1, double bc2)
{
    double g = g32;
    double m1 = hp->beta1 * (double)*m + (1.0 - hp->beta1) * g;
    double v1 = hp->beta2 * (double)*v + (1.0 - hp->beta2) * (g * g);
    double mhat = m1 / bc1;
    double vhat = v1 / bc2;
    double upd = mhat / (sqrt(vhat) + hp->eps);
    double th = (double)*theta * (1.0 - hp->lr * hp->weight_decay) - hp->lr * upd;
    *m = (float)m1;
    *v = (float)v1;
    *theta = (float)th;
}

static double bias_correction(double beta, int64_t t)
{
    return 1.0 - pow(beta, (double)t);
}

/*
 * Two extensions of the reduce, for data-parallel layouts beyond one flat
 * group and for more than one micro-batch per step:
 *
 *  - Hybrid sharding (CS231n "Large-Scale Distributed Training" notes, 4.4:
 *    N = M x K GPUs, sharded inside each group of K, replicated across the
 *    M groups).  The gradient is reduced inside each group first, then
 *    across groups.  Order: ranks m*K .. m*K+K-1 form group m; each group's
 *    partials are summed in rank order, then the M group sums in group
 *    order, all in double.  K = N (one group) and K = 1 both give the flat
 *    rank-order fold.
 *
 *  - Gradient accumulation over G micro-batches ("并行训练优化、MoE扩展与系统
 *    瓶颈", 3.1: the effective batch is micro-batch x data-parallel size x
 *    accumulation steps).  The gradient is the mean over all N x G
 *    micro-batch gradients.  An fp32 accumulator holds the running sum of
 *    the earlier micro-batches' reductions: after micro-batch j it is
 *    fp32(acc + s_j) (for j = 0 just fp32(s_0)); the last micro-batch's
 *    step uses g = fp32((acc + s_last) / (N G)), sums in double.
 */
static double grouped_sum(const void *const *partials, int n_ranks, int group, int gdt,
                          int64_t i)
{
    double s = 0.0;
    for (int m = 0; m < n_ranks / group; ++m) {
        double t = partial_at(partials[m * group], gdt, i);
        for (int k = 1; k < group; ++k)
            t = t + partial_at(partials[m * group + k], gdt, i);
        s = (m == 0) ? t : s + t;
    }
    return s;
}

static float reduce_ex_one(const void *const *partials, int n_ranks, int group, int gdt,
                           const float *acc, int64_t micro_batches, int64_t i)
{
    double s = grouped_sum(partials, n_ranks, group, gdt, i);
    if (acc)
        s = (double)acc[i] + s;
    return (float)(s / ((double)n_ranks * (double)micro_batches));
}

/*
 * The 12-bytes-per-parameter ledger ("并行训练优化、MoE扩展与系统瓶颈", 2.2.9:
 * everything but the master weights in BF16 comes to about 12 bytes per
 * parameter; the same 2 + 2 + 8 split sizes the capacity table of Lecture 8,
 * Slide 28): bf16 parameter and gradient, fp32 master, bf16 Adam m and v.
 * The update is the AdamW above with the moments read from and rounded back
 * to bf16: m' and v' (double) are each rounded once, to nearest even, straight
 * to bf16.
 *
 * Rounding a double to bf16 (8 significant bits, fp32's exponent range):
 * write |d| = f 2^E with 1/2 <= f < 1; the candidates are the multiples of
 * 2^(E-8), or of 2^-133 below the normal range (bf16 subnormals); rint()
 * rounds the scaled value to the nearest integer, ties to even, exactly.
 * Results above the largest finite bf16 (0x7F7F = (2^8 - 1) 2^120) become inf.
 */
uint16_t oracle_bf16_from_double(double d)
{
    if (isnan(d)) {
        float f = (float)d;                       /* keeps the sign; quiet */
        uint32_t u;
        memcpy(&u, &f, 4);
        return (uint16_t)((u >> 16) | 0x0040u);
    }
    double a = fabs(d);
    double r = 0.0;
    if (a != 0.0 && !isinf(a)) {
        int E;
        frexp(a, &E);                             /* a = f 2^E, 1/2 <= f < 1 */
        int q = E - 8;                            /* spacing 2^q of 8-bit significands */
        if (q < -133)
            q = -133;                             /* subnormal spacing */
        r = ldexp(rint(ldexp(a, -q)), q);         /* exact scaling, one rounding */
        if (r > ldexp(255.0, 120))
            r = INFINITY;
    } else {
        r = a;
    }
    float f = (float)(signbit(d) ? -r : r);       /* exact: r has <= 8 significant bits */
    uint32_t u;
    memcpy(&u, &f, 4);
    return (uint16_t)(u >> 16);
}

void oracle_bf16_from_double_array(const double *in, int64_t n, uint16_t *out)
{
#pragma omp parallel for schedule(static) if (n > ORACLE_PAR_MIN)
    for (int64_t i = 0; i < n; ++i)
        out[i] = oracle_bf16_from_double(in[i]);
}

/* ---- array entry points --------------------------------------------- */

/* g_out[i] = fp32( (p_0[i] + p_1[i] + ... + p_{N-1}[i]) / N ), i in [0, n). */
void oracle_reduce(const void *const *partials, int n_ranks, int gdt, int64_t n, float *g_out)
{
#pragma omp parallel for schedule(static) if (n > ORACLE_PAR_MIN)
    for (int64_t i = 0; i < n; ++i)
        g_out[i] = reduce_one(partials, n_ranks, gdt, i);
}

/* One AdamW update of n elements in place, from an fp32 gradient. */
void oracle_adamw(const float *g, float *master, float *m, float *v, int64_t n,
                  const oracle_hparams *hp)
{
    double bc1 = bias_correction(hp->beta1, hp->step);
    double bc2 = bias_correction(hp->beta2, hp->step);
#pragma omp parallel for schedule(static) if (n > ORACLE_PAR_MIN)
    for (int64_t i = 0; i < n; ++i)
        adamw_one(g[i], &master[i], &m[i], &v[i], hp, bc1, bc2);
}

/* The whole shard step: reduce, AdamW, bf16 parameter (in shard order). */
void oracle_shard_step(const void *const *partials, int n_ranks, int gdt, int64_t n,
                       float *master, float *m, float *v, const oracle_hparams *hp,
                       uint16_t *param_out)
{
    double bc1 = bias_correction(hp->beta1, hp->step);
    double bc2 = bias_correction(hp->beta2, hp->step);
#pragma omp parallel for schedule(static) if (n > ORACLE_PAR_MIN)
    for (int64_t i = 0; i < n; ++i) {
        float g = reduce_one(partials, n_ranks, gdt, i);
        adamw_one(g, &master[i], &m[i], &v[i], hp, bc1, bc2);
        if (param_out)
            param_out[i] = oracle_bf16_round(master[i]);
    }
}

/* g_out[i] = fp32(((acc[i] if acc) + grouped sum) / (N * micro_batches)). */
void oracle_reduce_ex(const void *const *partials, int n_ranks, int group, int gdt,
                      const float *acc, int64_t micro_batches, int64_t n, float *g_out)
{
#pragma omp parallel for schedule(static) if (n > ORACLE_PAR_MIN)
    for (int64_t i = 0; i < n; ++i)
        g_out[i] = reduce_ex_one(partials, n_ranks, group, gdt, acc, micro_batches, i);
}

/* One non-final micro-batch: acc[i] = fp32((reset ? 0 : acc[i]) + grouped sum). */
void oracle_accumulate(const void *const *partials, int n_ranks, int group, int gdt,
                       int64_t n, float *acc, int reset)
{
#pragma omp parallel for schedule(static) if (n > ORACLE_PAR_MIN)
    for (int64_t i = 0; i < n; ++i) {
        double s = grouped_sum(partials, n_ranks, group, gdt, i);
        acc[i] = reset ? (float)s : (float)((double)acc[i] + s);
    }
}

/* The whole shard step with the extended reduce. */
void oracle_shard_step_ex(const void *const *partials, int n_ranks, int group, int gdt,
                          const float *acc, int64_t micro_batches, int64_t n, float *master,
                          float *m, float *v, const oracle_hparams *hp, uint16_t *param_out)
{
    double bc1 = bias_correction(hp->beta1, hp->step);
    double bc2 = bias_correction(hp->beta2, hp->step);
#pragma omp parallel for schedule(static) if (n > ORACLE_PAR_MIN)
    for (int64_t i = 0; i < n; ++i) {
        float g = reduce_ex_one(partials, n_ranks, group, gdt, acc, micro_batches, i);
        adamw_one(g, &master[i], &m[i], &v[i], hp, bc1, bc2);
        if (param_out)
            param_out[i] = oracle_bf16_round(master[i]);
    }
}

/* The shard step on the 12-byte state: m, v are bf16 bit patterns. */
void oracle_shard_step_bf16m(const void *const *partials, int n_ranks, int gdt, int64_t n,
                             float *master, uint16_t *m, uint16_t *v, const oracle_hparams *hp,
                             uint16_t *param_out)
{
    double bc1 = bias_correction(hp->beta1, hp->step);
    double bc2 = bias_correction(hp->beta2, hp->step);
#pragma omp parallel for schedule(static) if (n > ORACLE_PAR_MIN)
    for (int64_t i = 0; i < n; ++i) {
        double g = reduce_one(partials, n_ranks, gdt, i);
        double m1 = hp->beta1 * bf16_value(m[i]) + (1.0 - hp->beta1) * g;
        double v1 = hp->beta2 * bf16_value(v[i]) + (1.0 - hp->beta2) * (g * g);
        double mhat = m1 / bc1;
        double vhat = v1 / bc2;
        double upd = mhat / (sqrt(vhat) + hp->eps);
        double th = (double)master[i] * (1.0 - hp->lr * hp->weight_decay) - hp->lr * upd;
        m[i] = oracle_bf16_from_double(m1);
        v[i] = oracle_bf16_from_double(v1);
        master[i] = (float)th;
        if (param_out)
            param_out[i] = oracle_bf16_round(master[i]);
    }
}

/*
 * Pure-bf16 state with a compensated parameter update.  Lecture 8, Slide 28
 * sizes its ZeRO capacity table with a "pure-BF16/Kahan" ledger and gives
 * no formula.  Reading: the bf16 parameter (in its slot) is the only copy
 * of the weight, there is no fp32 master; a bf16 buffer c holds the part of
 * earlier increments that the bf16 parameter has not absorbed yet.  The
 * increment is added by Kahan's compensated summation (Kahan 1965; applied
 * to bf16 weight updates by Zamirai et al., "Revisiting BFloat16 Training"):
 *     y      = d + c
 *     theta' = bf16(theta + y)
 *     c'     = bf16(y - (theta' - theta))
 * with d the AdamW increment -lr (u + wd theta), u = mhat / (sqrt(vhat) + eps)
 * from bf16 m, v as in the 12-byte step.  Arithmetic in double; each stored
 * value (theta', c', m', v') is rounded once to nearest-even bf16.
 */
static void kahan_one(uint16_t *theta, uint16_t *comp, double d)
{
    double th = bf16_value(*theta);
    double y = d + bf16_value(*comp);
    uint16_t t1 = oracle_bf16_from_double(th + y);
    double moved = bf16_value(t1) - th;           /* what theta absorbed */
    *comp = oracle_bf16_from_double(y - moved);
    *theta = t1;
}

/* The compensated add alone: (theta, c) += delta, element by element. */
void oracle_kahan_add(uint16_t *theta, uint16_t *comp, const double *delta, int64_t n)
{
#pragma omp parallel for schedule(static) if (n > ORACLE_PAR_MIN)
    for (int64_t i = 0; i < n; ++i)
        kahan_one(&theta[i], &comp[i], delta[i]);
}

/* The shard step on the pure-bf16 state: theta (the parameters in shard
 * order), comp, m, v are bf16 bit patterns, updated in place. */
void oracle_shard_step_kahan(const void *const *partials, int n_ranks, int gdt, int64_t n,
                             uint16_t *theta, uint16_t *comp, uint16_t *m, uint16_t *v,
                             const oracle_hparams *hp)
{
    double bc1 = bias_correction(hp->beta1, hp->step);
    double bc2 = bias_correction(hp->beta2, hp->step);
#pragma omp parallel for schedule(static) if (n > ORACLE_PAR_MIN)
    for (int64_t i = 0; i < n; ++i) {
        double g = reduce_one(partials, n_ranks, gdt, i);
        double m1 = hp->beta1 * bf16_value(m[i]) + (1.0 - hp->beta1) * g;
        double v1 = hp->beta2 * bf16_value(v[i]) + (1.0 - hp->beta2) * (g * g);
        double mhat = m1 / bc1;
        double vhat = v1 / bc2;
        double upd = mhat / (sqrt(vhat) + hp->eps);
        double d = -hp->lr * (upd + hp->weight_decay * bf16_value(theta[i]));
        m[i] = oracle_bf16_from_double(m1);
        v[i] = oracle_bf16_from_double(v1);
        kahan_one(&theta[i], &comp[i], d);
    }
}

/*
 * Shard geometry: the pieces of rank `rank`'s segment, one per tensor it
 * touches.  seg[4*j + 0..3] = {tensor id, element offset inside the tensor,
 * offset inside the shard, length}.  Returns the number of pieces (at most
 * cap are written) and stores the shard length S in *shard_len.
 */
int64_t oracle_shard_segments(const int64_t *numels, int n_tensors, int n_ranks, int rank,
                              int64_t *seg, int64_t cap, int64_t *shard_len)
{
    int64_t total = 0;
    for (int t = 0; t < n_tensors; ++t)
        total += numels[t];
    int64_t S = (total + n_ranks - 1) / n_ranks;
    int64_t lo = (int64_t)rank * S, hi = lo + S;
    if (lo > total) lo = total;
    if (hi > total) hi = total;
    *shard_len = S;
    int64_t count = 0, start = 0;
    for (int t = 0; t < n_tensors; ++t) {
        int64_t a = start, b = start + numels[t];
        int64_t x = a > lo ? a : lo, y = b < hi ? b : hi;
        if (x < y) {
            if (count < cap) {
                seg[4 * count + 0] = t;
                seg[4 * count + 1] = x - a;
                seg[4 * count + 2] = x - lo;
                seg[4 * count + 3] = y - x;
            }
            ++count;
        }
        start = b;
    }
    return count;
}

void oracle_set_threads(int n)
{
#ifdef _OPENMP
    omp_set_num_threads(n);
#else
    (void)n;
#endif
}

int oracle_max_threads(void)
{
#ifdef _OPENMP
    return omp_get_max_threads();
#else
    return 1;
#endif
}
