/*
 * afd_oracle.c -- TEST INFRASTRUCTURE ONLY.
 *
 * A plain, slow, fp64 CPU reference for the expert (FFN) side of an
 * attention-FFN-disaggregated MoE layer.  Only the test suite, the smoke
 * check and the CPU-baseline leg of the benchmark may load this library;
 * the product path never calls it and shares no code with it.
 *
 * What is computed (sources: "FastAFD" structured summary, System Design
 * items 1-3 and the legend of Eq. (3); vLLM AFD plugin blog, "FFN service"):
 * the FFN side receives token hidden states together with the top-k routing
 * metadata chosen on the attention side (expert ids and weights), runs the
 * routed experts' FFNs (grouped GEMMs plus the activation) and returns the
 * combined output per token.  The pages do not write the formula out; the
 * plain reading used here is the standard SwiGLU MoE layer
 *
 *     y_t = sum_{k : ids[t,k] >= 0} w[t,k] * FFN_{ids[t,k]}(x_t)  [+ FFN_S(x_t)]
 *     FFN_e(x) = Wd_e^T ( silu(Wg_e^T x) .* (Wu_e^T x) ),  silu(z) = z/(1+e^-z)
 *
 * with Wg_e, Wu_e stored [H, I] and Wd_e stored [I, H] (row-major, stacked
 * over experts), id -1 meaning "expert not on this GPU", duplicate ids
 * counting as separate assignments, and the routing weights used exactly as
 * given (no re-normalisation: routing is done on the attention side).
 *
 * Inputs are decoded exactly to fp64: fp32 as is, bf16 by widening its bit
 * pattern, block-FP8 (OCP E4M3FN codes) as code value times its fp32 block
 * scale (1x128 groups along H for activations, 128x128 blocks for weights).
 * The intermediate activation is kept exact (no re-quantisation).
 *
 * W8A8 (the "W8A8" expert precision of the vLLM AFD plugin blog's decode
 * benchmark; the page names only "W8A8", so the format is a reading): int8
 * codes, symmetric, weights with one fp32 scale per output channel (per
 * column of Wg, Wu [H, I] and of Wd [I, H]), activations with one fp32 scale
 * per token; a value is code times its scale, decoded exactly to fp64 here.
 *
 * Dispatch (the expert-major permutation the GPU builds) is given by its
 * definition: per-expert counts, exclusive prefix sums, and the flat
 * assignment indices t*K+k listed expert by expert in ascending flat order.
 *
 * Parity of the expert arithmetic is pinned by the CPU tests against a dense
 * brute-force formulation, library matrix products and invariants; the
 * pages print no worked example.
 */
#include <math.h>
#include <pthread.h>
#include <stdint.h>
#include <stdlib.h>
#include <string.h>
#include <unistd.h>

enum { ORACLE_F32 = 0, ORACLE_BF16 = 1, ORACLE_FP8 = 2, ORACLE_W8A8 = 3 };

typedef struct {
    int32_t T, H, I, E, K;   /* tokens, hidden, intermediate, experts, top-k     */
    int32_t shared_inter;    /* 0: no shared expert; else its intermediate size  */
    int32_t dtype;           /* ORACLE_F32 / ORACLE_BF16 / ORACLE_FP8 / ORACLE_W8A8 */
    const void *hidden;      /* [T,H] f32 | bf16 bits | e4m3 codes | int8 codes   */
    const float *hidden_scales; /* FP8: [T, H/128]; W8A8: [T] (one per token)     */
    const int32_t *ids;      /* [T,K], -1 = not here                              */
    const float *weights;    /* [T,K]                                             */
    const void *w_gate, *w_up, *w_down;   /* [E,H,I], [E,H,I], [E,I,H]            */
    const float *s_gate, *s_up, *s_down;  /* FP8: [E,H/128,I/128] x2, [E,I/128,H/128];
                                             W8A8: [E,I] x2, [E,H] (per output column) */
    const void *sh_gate, *sh_up, *sh_down;    /* shared: [H,Is], [H,Is], [Is,H]   */
    const float *sh_s_gate, *sh_s_up, *sh_s_down;
} afd_oracle_problem;

/* ---- exact decoders --------------------------------------------------- */

double afd_oracle_bf16_to_f64(uint16_t b)
{
    /* bf16 is the upper half of an IEEE binary32 pattern. */
    uint32_t u = (uint32_t)b << 16;
    float f;
    memcpy(&f, &u, sizeof f);
    return (double)f;
}

double afd_oracle_e4m3_to_f64(uint8_t c)
{
    /* OCP E4M3FN: 1 sign, 4 exponent (bias 7), 3 mantissa bits; no
     * infinities; S.1111.111 is NaN; exponent field 0 is subnormal. */
    int s = c >> 7, e = (c >> 3) & 0xF, m = c & 7;
    double v;
    if (e == 15 && m == 7)
        return NAN;
    if (e == 0)
        v = ldexp((double)m / 8.0, -6);
    else
        v = ldexp(1.0 + (double)m / 8.0, e - 7);
    return s ? -v : v;
}

double afd_oracle_i8_to_f64(uint8_t raw)
{
    /* two's complement: bytes 128..255 are -128..-1 */
    return (double)(raw < 128 ? (int)raw : (int)raw - 256);
}

/* Element (r, c) of a row-major [rows, cols] matrix, decoded.  For FP8,
 * `scales` is the [rows/128, cols/128] block-scale grid of that matrix; for
 * W8A8 its [cols] per-column scales. */
static double elem(int dtype, const void *base, size_t off, int cols,
                   const float *scales, int r, int c)
{
    size_t i = off + (size_t)r * cols + c;
    switch (dtype) {
    case ORACLE_F32:
        return (double)((const float *)base)[i];
    case ORACLE_BF16:
        return afd_oracle_bf16_to_f64(((const uint16_t *)base)[i]);
    case ORACLE_W8A8:
        return afd_oracle_i8_to_f64(((const uint8_t *)base)[i]) * (double)scales[c];
    default: {
        int bc = cols / 128;
        return afd_oracle_e4m3_to_f64(((const uint8_t *)base)[i]) *
               (double)scales[(size_t)(r / 128) * bc + (c / 128)];
    }
    }
}

/* ---- dispatch ----------------------------------------------------------- */

/* Returns 0, or -1 when an id lies outside [-1, E). */
int afd_oracle_dispatch(int32_t T, int32_t K, int32_t E, const int32_t *ids,
                        int32_t *counts, int32_t *offsets,
                        int32_t *sorted_assign, int32_t *row_of)
{
    int64_t n = (int64_t)T * K;
    for (int64_t f = 0; f < n; ++f)
        if (ids[f] < -1 || ids[f] >= E)
            return -1;
    for (int e = 0; e < E; ++e)
        counts[e] = 0;
    for (int64_t f = 0; f < n; ++f)
        if (ids[f] >= 0)
            counts[ids[f]] += 1;
    offsets[0] = 0;
    for (int e = 0; e < E; ++e)
        offsets[e + 1] = offsets[e] + counts[e];
    int32_t *cursor = (int32_t *)malloc(sizeof(int32_t) * (E > 0 ? E : 1));
    if (!cursor)
        return -2;
    for (int e = 0; e < E; ++e)
        cursor[e] = offsets[e];
    for (int64_t f = 0; f < n; ++f) {
        int e = ids[f];
        if (e < 0) {
            row_of[f] = -1;
            continue;
        }
        sorted_assign[cursor[e]] = (int32_t)f;
        row_of[f] = cursor[e];
        cursor[e] += 1;
    }
    free(cursor);
    return 0;
}

/* ---- one expert FFN ------------------------------------------------------ */

typedef struct {
    int dtype, H, Is;
    const void *wg, *wu, *wd;
    size_t og, ou, od;             /* element offset of this expert's matrices */
    const float *sg, *su, *sd;     /* this expert's scales (FP8 grids, W8A8 columns) */
} ffn_view;

/* f[H] = Wd^T (silu(Wg^T x) .* (Wu^T x)), all in fp64. g, u: scratch [Is]. */
static void ffn(const ffn_view *v, const double *x, double *g, double *u, double *f)
{
    int H = v->H, Is = v->Is;
    for (int i = 0; i < Is; ++i)
        g[i] = u[i] = 0.0;
    for (int h = 0; h < H; ++h) {
        double xh = x[h];
        for (int i = 0; i < Is; ++i) {
            g[i] += xh * elem(v->dtype, v->wg, v->og, Is, v->sg, h, i);
            u[i] += xh * elem(v->dtype, v->wu, v->ou, Is, v->su, h, i);
        }
    }
    for (int i = 0; i < Is; ++i) {
        double z = g[i];
        g[i] = (z / (1.0 + exp(-z))) * u[i]; /* silu(gate) * up */
    }
    for (int h = 0; h < H; ++h)
        f[h] = 0.0;
    for (int i = 0; i < Is; ++i) {
        double a = g[i];
        for (int h = 0; h < H; ++h)
            f[h] += a * elem(v->dtype, v->wd, v->od, H, v->sd, i, h);
    }
}

static ffn_view routed_view(const afd_oracle_problem *p, int e)
{
    ffn_view v;
    int H = p->H, I = p->I;
    v.dtype = p->dtype;
    v.H = H;
    v.Is = I;
    v.wg = p->w_gate;
    v.wu = p->w_up;
    v.wd = p->w_down;
    v.og = v.ou = v.od = (size_t)e * H * I;
    if (p->dtype == ORACLE_FP8) {
        size_t sblk = (size_t)(H / 128) * (I / 128);
        v.sg = p->s_gate + (size_t)e * sblk;
        v.su = p->s_up + (size_t)e * sblk;
        v.sd = p->s_down + (size_t)e * sblk;
    } else if (p->dtype == ORACLE_W8A8) {
        v.sg = p->s_gate + (size_t)e * I;
        v.su = p->s_up + (size_t)e * I;
        v.sd = p->s_down + (size_t)e * H;
    } else {
        v.sg = v.su = v.sd = NULL;
    }
    return v;
}

static ffn_view shared_view(const afd_oracle_problem *p)
{
    ffn_view v;
    v.dtype = p->dtype;
    v.H = p->H;
    v.Is = p->shared_inter;
    v.wg = p->sh_gate;
    v.wu = p->sh_up;
    v.wd = p->sh_down;
    v.og = v.ou = v.od = 0;
    v.sg = p->sh_s_gate;
    v.su = p->sh_s_up;
    v.sd = p->sh_s_down;
    return v;
}

/* y = sum_k w[t,k] FFN_{ids[t,k]}(x_t) in k order, then + FFN_S(x_t). */
static void token_output(const afd_oracle_problem *p, int t, double *x, double *g,
                         double *u, double *f, double *y)
{
    int H = p->H, K = p->K;
    for (int h = 0; h < H; ++h) {
        size_t i = (size_t)t * H + h;
        switch (p->dtype) {
        case ORACLE_F32:
            x[h] = (double)((const float *)p->hidden)[i];
            break;
        case ORACLE_BF16:
            x[h] = afd_oracle_bf16_to_f64(((const uint16_t *)p->hidden)[i]);
            break;
        case ORACLE_W8A8:
            x[h] = afd_oracle_i8_to_f64(((const uint8_t *)p->hidden)[i]) *
                   (double)p->hidden_scales[t];
            break;
        default:
            x[h] = afd_oracle_e4m3_to_f64(((const uint8_t *)p->hidden)[i]) *
                   (double)p->hidden_scales[(size_t)t * (H / 128) + h / 128];
        }
    }
    for (int h = 0; h < H; ++h)
        y[h] = 0.0;
    for (int k = 0; k < K; ++k) {
        int e = p->ids[(size_t)t * K + k];
        if (e < 0)
            continue;
        double w = (double)p->weights[(size_t)t * K + k];
        ffn_view v = routed_view(p, e);
        ffn(&v, x, g, u, f);
        for (int h = 0; h < H; ++h)
            y[h] += w * f[h];
    }
    if (p->shared_inter > 0) {
        ffn_view v = shared_view(p);
        ffn(&v, x, g, u, f);
        for (int h = 0; h < H; ++h)
            y[h] += f[h];
    }
}

typedef struct {
    const afd_oracle_problem *p;
    const int32_t *tokens;
    int32_t ntok;
    double *out;
    int tid, nthreads;
    int status;
} worker_arg;

static void *worker(void *argp)
{
    worker_arg *a = (worker_arg *)argp;
    const afd_oracle_problem *p = a->p;
    int H = p->H;
    int Imax = p->I > p->shared_inter ? p->I : p->shared_inter;
    double *x = (double *)malloc(sizeof(double) * H);
    double *f = (double *)malloc(sizeof(double) * H);
    double *g = (double *)malloc(sizeof(double) * (Imax > 0 ? Imax : 1));
    double *u = (double *)malloc(sizeof(double) * (Imax > 0 ? Imax : 1));
    a->status = 0;
    if (!x || !f || !g || !u) {
        a->status = -2;
    } else {
        for (int j = a->tid; j < a->ntok; j += a->nthreads)
            token_output(p, a->tokens[j], x, g, u, f, a->out + (size_t)j * H);
    }
    free(x);
    free(f);
    free(g);
    free(u);
    return NULL;
}

/*
 * out[j, :] = y_{tokens[j]} for j < ntok, fp64, row-major [ntok, H].
 * nthreads <= 0 uses every online CPU.  Returns 0, -1 on a bad argument or
 * id, -2 when memory or threads cannot be had.
 */
int afd_oracle_forward(const afd_oracle_problem *p, int32_t ntok, const int32_t *tokens,
                       double *out, int32_t nthreads)
{
    if (!p || p->T < 0 || p->H <= 0 || p->I <= 0 || p->E <= 0 || p->K <= 0 ||
        p->shared_inter < 0 || p->dtype < ORACLE_F32 || p->dtype > ORACLE_W8A8 || ntok < 0 ||
        (ntok > 0 && (!tokens || !out)))
        return -1;
    if (p->dtype == ORACLE_FP8 && (p->H % 128 || p->I % 128 || p->shared_inter % 128))
        return -1;
    for (int j = 0; j < ntok; ++j) {
        if (tokens[j] < 0 || tokens[j] >= p->T)
            return -1;
        for (int k = 0; k < p->K; ++k) {
            int e = p->ids[(size_t)tokens[j] * p->K + k];
            if (e < -1 || e >= p->E)
                return -1;
        }
    }
    if (nthreads <= 0)
        nthreads = (int)sysconf(_SC_NPROCESSORS_ONLN);
    if (nthreads > ntok)
        nthreads = ntok > 0 ? ntok : 1;
    pthread_t *th = (pthread_t *)malloc(sizeof(pthread_t) * nthreads);
    worker_arg *args = (worker_arg *)malloc(sizeof(worker_arg) * nthreads);
    if (!th || !args) {
        free(th);
        free(args);
        return -2;
    }
    int rc = 0, started = 0;
    for (int i = 0; i < nthreads; ++i) {
        args[i].p = p;
        args[i].tokens = tokens;
        args[i].ntok = ntok;
        args[i].out = out;
        args[i].tid = i;
        args[i].nthreads = nthreads;
        args[i].status = 0;
        if (pthread_create(&th[i], NULL, worker, &args[i]) != 0) {
            rc = -2;
            break;
        }
        started++;
    }
    for (int i = 0; i < started; ++i) {
        pthread_join(th[i], NULL);
        if (args[i].status)
            rc = args[i].status;
    }
    free(th);
    free(args);
    return rc;
}
