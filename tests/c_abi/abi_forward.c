/*
 * abi_forward.c -- the C ABI of include/afd_ffn.h used from plain C, with no
 * Python or torch in the process (test infrastructure: built by the build
 * step, run by tests/test_gpu_c_abi.py).
 *
 * One small layer (ragged T, a shared expert of another width than the routed
 * experts, some slots routed elsewhere with id -1) in bf16 or block-FP8:
 * create a handle from device weights, run one forward on a HIP stream of the
 * program's own, and compare against the fp64 oracle (oracle/afd_oracle.c,
 * linked directly): the dispatch bit for bit (afd_ffn_debug_dispatch against
 * afd_oracle_dispatch) and the outputs within the layer's tolerance
 * (max|out - ref| <= tol * max|ref|: 2e-2 bf16, 6e-2 block-FP8).  Also checks
 * that an oversized T is refused on the host with a message.
 *
 * Inputs are drawn as valid bit patterns from a seeded splitmix64 stream, so
 * no encoder is involved: bf16 values are the upper halves of fp32 draws,
 * e4m3 codes have exponent fields 4..9 (no NaN code), scales are positive
 * fp32 draws.
 *
 *   abi_forward bf16|fp8        exit 0: pass, 1: mismatch, 2: setup error
 */
#include <math.h>
#include <stdint.h>
#include <stdio.h>
#include <stdlib.h>
#include <string.h>

#include <hip/hip_runtime_api.h>

#include "afd_ffn.h"

/* The oracle's problem description and entry points (oracle/afd_oracle.c). */
typedef struct {
    int32_t T, H, I, E, K, shared_inter, dtype;
    const void *hidden;
    const float *hidden_scales;
    const int32_t *ids;
    const float *weights;
    const void *w_gate, *w_up, *w_down;
    const float *s_gate, *s_up, *s_down;
    const void *sh_gate, *sh_up, *sh_down;
    const float *sh_s_gate, *sh_s_up, *sh_s_down;
} afd_oracle_problem;
int afd_oracle_dispatch(int32_t T, int32_t K, int32_t E, const int32_t *ids, int32_t *counts,
                        int32_t *offsets, int32_t *sorted_assign, int32_t *row_of);
int afd_oracle_forward(const afd_oracle_problem *p, int32_t ntok, const int32_t *tokens, double *out,
                       int32_t nthreads);

enum { T = 77, TMAX = 96, H = 256, I = 384, E = 6, K = 3, IS = 256 };

static uint64_t rng_state = 0x5eed0afd2024ull;

static uint64_t next_u64(void) /* splitmix64 */
{
    uint64_t z = (rng_state += 0x9e3779b97f4a7c15ull);
    z = (z ^ (z >> 30)) * 0xbf58476d1ce4e5b9ull;
    z = (z ^ (z >> 27)) * 0x94d049bb133111ebull;
    return z ^ (z >> 31);
}

static float uniform(float lo, float hi) { return lo + (hi - lo) * (float)((next_u64() >> 40) * 0x1.0p-24); }

static uint16_t bf16_draw(float lo, float hi) /* the upper half of an fp32 draw */
{
    float f = uniform(lo, hi);
    uint32_t u;
    memcpy(&u, &f, 4);
    return (uint16_t)(u >> 16);
}

static uint8_t e4m3_draw(void) /* sign, exponent field 4..9, any mantissa */
{
    uint64_t r = next_u64();
    return (uint8_t)(((r & 1) << 7) | ((4 + (r >> 1) % 6) << 3) | ((r >> 8) & 7));
}

#define CHECK_HIP(x)                                                                 \
    do {                                                                             \
        hipError_t e_ = (x);                                                         \
        if (e_ != hipSuccess) {                                                      \
            fprintf(stderr, "%s: %s\n", #x, hipGetErrorString(e_));                  \
            exit(2);                                                                 \
        }                                                                            \
    } while (0)

#define CHECK_AFD(x)                                                                 \
    do {                                                                             \
        afd_status s_ = (x);                                                         \
        if (s_ != AFD_OK) {                                                          \
            fprintf(stderr, "%s: %s (%s)\n", #x, afd_ffn_status_string(s_), afd_ffn_last_error()); \
            exit(2);                                                                 \
        }                                                                            \
    } while (0)

static void *to_device(const void *host, size_t bytes)
{
    void *d = NULL;
    CHECK_HIP(hipMalloc(&d, bytes ? bytes : 16));
    if (host && bytes) CHECK_HIP(hipMemcpy(d, host, bytes, hipMemcpyHostToDevice));
    return d;
}

int main(int argc, char **argv)
{
    const int fp8 = argc > 1 && strcmp(argv[1], "fp8") == 0;
    if (argc < 2 || (!fp8 && strcmp(argv[1], "bf16") != 0)) {
        fprintf(stderr, "usage: abi_forward bf16|fp8\n");
        return 2;
    }
    const size_t es = fp8 ? 1 : 2;
    const size_t n_wgu = (size_t)E * H * I, n_wd = (size_t)E * I * H;
    const size_t n_sgu = (size_t)IS * H;

    /* inputs (host) */
    void *hidden = malloc((size_t)T * H * es), *wg = malloc(n_wgu * es), *wu = malloc(n_wgu * es),
         *wd = malloc(n_wd * es), *shg = malloc(n_sgu * es), *shu = malloc(n_sgu * es),
         *shd = malloc(n_sgu * es);
    void *bufs[] = {hidden, wg, wu, wd, shg, shu, shd};
    const size_t counts_[] = {(size_t)T * H, n_wgu, n_wgu, n_wd, n_sgu, n_sgu, n_sgu};
    for (int b = 0; b < 7; ++b)
        for (size_t i = 0; i < counts_[b]; ++i) {
            if (fp8)
                ((uint8_t *)bufs[b])[i] = e4m3_draw();
            else
                ((uint16_t *)bufs[b])[i] = b == 0 ? bf16_draw(-1.0f, 1.0f) : bf16_draw(-0.06f, 0.06f);
        }
    /* block-FP8 scales: activations per 1x128 group, weights per 128x128 block */
    const int hb = H / 128, ib = I / 128, isb = IS / 128;
    float *xs = malloc(sizeof(float) * T * hb), *sg = malloc(sizeof(float) * E * hb * ib),
          *su = malloc(sizeof(float) * E * hb * ib), *sd = malloc(sizeof(float) * E * ib * hb),
          *ssg = malloc(sizeof(float) * hb * isb), *ssu = malloc(sizeof(float) * hb * isb),
          *ssd = malloc(sizeof(float) * isb * hb);
    for (int i = 0; i < T * hb; ++i) xs[i] = uniform(0.05f, 0.2f);
    for (int i = 0; i < E * hb * ib; ++i) {
        sg[i] = uniform(0.002f, 0.01f);
        su[i] = uniform(0.002f, 0.01f);
        sd[i] = uniform(0.002f, 0.01f);
    }
    for (int i = 0; i < hb * isb; ++i) {
        ssg[i] = uniform(0.002f, 0.01f);
        ssu[i] = uniform(0.002f, 0.01f);
        ssd[i] = uniform(0.002f, 0.01f);
    }
    /* routing: K distinct experts per token, about one slot in six routed elsewhere (-1) */
    int32_t ids[T * K];
    float wts[T * K];
    for (int t = 0; t < T; ++t)
        for (int k = 0; k < K; ++k) {
            int e;
            int again;
            do {
                e = (int)(next_u64() % E);
                again = 0;
                for (int j = 0; j < k; ++j) again |= ids[t * K + j] == e;
            } while (again);
            ids[t * K + k] = e;
            wts[t * K + k] = uniform(0.05f, 0.6f);
        }
    for (int f = 0; f < T * K; ++f)
        if (next_u64() % 6 == 0) ids[f] = -1;

    /* device copies, handle, one forward on the program's stream */
    afd_ffn_config cfg;
    memset(&cfg, 0, sizeof cfg);
    cfg.hidden = H;
    cfg.inter = I;
    cfg.num_experts = E;
    cfg.top_k = K;
    cfg.max_tokens = TMAX;
    cfg.shared_inter = IS;
    cfg.dtype = fp8 ? AFD_DTYPE_FP8_BLOCK : AFD_DTYPE_BF16;
    cfg.device = 0;
    cfg.w_gate = to_device(wg, n_wgu * es);
    cfg.w_up = to_device(wu, n_wgu * es);
    cfg.w_down = to_device(wd, n_wd * es);
    cfg.sh_gate = to_device(shg, n_sgu * es);
    cfg.sh_up = to_device(shu, n_sgu * es);
    cfg.sh_down = to_device(shd, n_sgu * es);
    if (fp8) {
        cfg.s_gate = to_device(sg, sizeof(float) * E * hb * ib);
        cfg.s_up = to_device(su, sizeof(float) * E * hb * ib);
        cfg.s_down = to_device(sd, sizeof(float) * E * ib * hb);
        cfg.sh_s_gate = to_device(ssg, sizeof(float) * hb * isb);
        cfg.sh_s_up = to_device(ssu, sizeof(float) * hb * isb);
        cfg.sh_s_down = to_device(ssd, sizeof(float) * isb * hb);
    }
    CHECK_AFD(afd_ffn_validate_config(&cfg));
    afd_ffn_t *h = NULL;
    CHECK_AFD(afd_ffn_create(&cfg, &h));
    void *d_hidden = to_device(hidden, (size_t)T * H * es);
    float *d_xs = fp8 ? to_device(xs, sizeof(float) * T * hb) : NULL;
    int32_t *d_ids = to_device(ids, sizeof ids);
    float *d_wts = to_device(wts, sizeof wts);
    void *d_out = to_device(NULL, (size_t)T * H * 2);
    hipStream_t stream;
    CHECK_HIP(hipStreamCreate(&stream));
    CHECK_AFD(afd_ffn_forward(h, T, d_hidden, d_xs, d_ids, d_wts, d_out, stream));
    int32_t *d_counts = to_device(NULL, sizeof(int32_t) * E), *d_offsets = to_device(NULL, sizeof(int32_t) * (E + 1)),
            *d_sa = to_device(NULL, sizeof(int32_t) * T * K), *d_row = to_device(NULL, sizeof(int32_t) * T * K);
    CHECK_AFD(afd_ffn_debug_dispatch(h, d_counts, d_offsets, d_sa, d_row, stream));
    CHECK_HIP(hipStreamSynchronize(stream));

    /* an oversized batch is refused on the host, with a message */
    const afd_status big = afd_ffn_forward(h, TMAX + 1, d_hidden, d_xs, d_ids, d_wts, d_out, stream);
    const int refused = big == AFD_ERR_INVALID_ARG && strlen(afd_ffn_last_error()) > 0;

    uint16_t out[T * H];
    int32_t counts[E], offsets[E + 1], sa[T * K], row_of[T * K];
    CHECK_HIP(hipMemcpy(out, d_out, sizeof out, hipMemcpyDeviceToHost));
    CHECK_HIP(hipMemcpy(counts, d_counts, sizeof counts, hipMemcpyDeviceToHost));
    CHECK_HIP(hipMemcpy(offsets, d_offsets, sizeof offsets, hipMemcpyDeviceToHost));
    CHECK_HIP(hipMemcpy(sa, d_sa, sizeof sa, hipMemcpyDeviceToHost));
    CHECK_HIP(hipMemcpy(row_of, d_row, sizeof row_of, hipMemcpyDeviceToHost));
    CHECK_AFD(afd_ffn_destroy(h));
    CHECK_HIP(hipStreamDestroy(stream));

    /* the oracle on the same host bytes */
    int32_t r_counts[E], r_offsets[E + 1], r_sa[T * K], r_row[T * K];
    if (afd_oracle_dispatch(T, K, E, ids, r_counts, r_offsets, r_sa, r_row) != 0) return 2;
    const int n = r_offsets[E];
    const int dispatch_exact = memcmp(counts, r_counts, sizeof counts) == 0 &&
                               memcmp(offsets, r_offsets, sizeof offsets) == 0 &&
                               memcmp(sa, r_sa, sizeof(int32_t) * n) == 0 && memcmp(row_of, r_row, sizeof r_row) == 0;
    afd_oracle_problem p;
    memset(&p, 0, sizeof p);
    p.T = T;
    p.H = H;
    p.I = I;
    p.E = E;
    p.K = K;
    p.shared_inter = IS;
    p.dtype = fp8 ? 2 : 1;
    p.hidden = hidden;
    p.hidden_scales = fp8 ? xs : NULL;
    p.ids = ids;
    p.weights = wts;
    p.w_gate = wg;
    p.w_up = wu;
    p.w_down = wd;
    p.sh_gate = shg;
    p.sh_up = shu;
    p.sh_down = shd;
    if (fp8) {
        p.s_gate = sg;
        p.s_up = su;
        p.s_down = sd;
        p.sh_s_gate = ssg;
        p.sh_s_up = ssu;
        p.sh_s_down = ssd;
    }
    double *ref = malloc(sizeof(double) * T * H);
    int32_t tokens[T];
    for (int t = 0; t < T; ++t) tokens[t] = t;
    if (afd_oracle_forward(&p, T, tokens, ref, 0) != 0) return 2;
    double err = 0.0, scale = 0.0;
    int finite = 1;
    for (int i = 0; i < T * H; ++i) {
        const uint32_t u = (uint32_t)out[i] << 16;
        float f;
        memcpy(&f, &u, 4);
        finite &= isfinite(f) != 0;
        err = fmax(err, fabs((double)f - ref[i]));
        scale = fmax(scale, fabs(ref[i]));
    }
    const double tol = fp8 ? 6e-2 : 2e-2;
    const int ok = finite && dispatch_exact && refused && scale > 0.0 && err <= tol * scale;
    printf("abi_forward %s: T=%d H=%d I=%d E=%d K=%d shared=%d routed=%d max|err|/max|ref| = %.3e (tol %.0e) "
           "dispatch %s, oversized T %s: %s\n",
           argv[1], T, H, I, E, K, IS, n, scale > 0.0 ? err / scale : 0.0, tol, dispatch_exact ? "exact" : "DIFFERS",
           refused ? "refused" : "NOT REFUSED", ok ? "PASS" : "FAIL");
    return ok ? 0 : 1;
}
