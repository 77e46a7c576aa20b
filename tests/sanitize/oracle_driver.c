/*
 * Runs the CPU oracles (oracle/dcnv4_oracle.c, oracle/fdattn_oracle.c) over
 * seeded small problems whose sampling locations include the awkward
 * values (NaN, +-inf, +-1e30, the exact borders -1 and H, values just
 * inside and outside them).  Built with AddressSanitizer and
 * UndefinedBehaviorSanitizer (float-cast-overflow included) by the test
 * suite; exits 0 and prints "ok <cases>" when no sanitizer fired and every
 * output is finite (the masks, logits and values here are finite).
 */
#include <math.h>
#include <stdint.h>
#include <stdio.h>
#include <stdlib.h>

int dcnv4o_output_size(int in, int kernel, int stride, int pad, int dil);
int dcnv4o_forward_ex(const float *value, const float *offset_mask, double *out, int N, int H, int W,
                      int kernel_h, int kernel_w, int stride_h, int stride_w, int pad_h, int pad_w, int dil_h,
                      int dil_w, int G, int Cg, float offset_scale, int remove_center, int P, int softmax,
                      int nthreads);
int dcnv4o_backward_ex(const float *value, const float *offset_mask, const float *grad_out, double *grad_value,
                       double *grad_offset_mask, int N, int H, int W, int kernel_h, int kernel_w, int stride_h,
                       int stride_w, int pad_h, int pad_w, int dil_h, int dil_w, int G, int Cg,
                       float offset_scale, int remove_center, int P, int softmax, int nthreads);
int fdao_forward(const float *value, const int *shapes, int L, const float *loc_attn, double *out, int N, int S,
                 int Q, int M, int D, int K, int P, int nthreads);
int fdao_backward(const float *value, const int *shapes, int L, const float *loc_attn, const float *grad_out,
                  double *grad_value, double *grad_loc_attn, int N, int S, int Q, int M, int D, int K, int P,
                  int nthreads);

static uint64_t state = 12345;

static uint32_t rnd(void)
{
    state = state * 6364136223846793005ull + 1442695040888963407ull;
    return (uint32_t)(state >> 33);
}

static float uniform(float lo, float hi)
{
    return lo + (hi - lo) * (float)(rnd() & 0xffffff) / 16777216.0f;
}

/* a location-like value: mostly ordinary, sometimes one of the awkward ones */
static float awkward(float size)
{
    switch (rnd() % 14) {
    case 0: return NAN;
    case 1: return INFINITY;
    case 2: return -INFINITY;
    case 3: return 1e30f;
    case 4: return -1e30f;
    case 5: return -1.0f;
    case 6: return size;
    case 7: return nextafterf(-1.0f, -2.0f);
    case 8: return nextafterf(size, 0.0f);
    case 9: return uniform(-50.0f, 50.0f);
    default: return uniform(-3.0f, 3.0f);
    }
}

static long cases = 0;

static void check_finite(const double *v, size_t n, const char *what)
{
    for (size_t i = 0; i < n; ++i)
        if (!isfinite(v[i])) {
            fprintf(stderr, "case %ld: %s[%zu] = %g\n", cases, what, i, v[i]);
            exit(1);
        }
}

static void conv_case(int N, int H, int W, int k, int stride, int pad, int dil, int G, int Cg, int rc, int sm)
{
    int Ho = dcnv4o_output_size(H, k, stride, pad, dil), Wo = dcnv4o_output_size(W, k, stride, pad, dil);
    if (Ho < 1 || Wo < 1)
        return;
    int K = k * k - rc, C = G * Cg, P = (3 * G * K + 7) / 8 * 8;
    size_t nv = (size_t)N * H * W * C, nom = (size_t)N * Ho * Wo * P, no = (size_t)N * Ho * Wo * C;
    float *v = malloc(nv * sizeof *v), *om = malloc(nom * sizeof *om), *go = malloc(no * sizeof *go);
    double *out = malloc(no * sizeof *out), *gv = malloc(nv * sizeof *gv), *gom = malloc(nom * sizeof *gom);
    for (size_t i = 0; i < nv; ++i)
        v[i] = uniform(-1.0f, 1.0f);
    for (size_t i = 0; i < no; ++i)
        go[i] = uniform(-1.0f, 1.0f);
    for (size_t px = 0; px < (size_t)N * Ho * Wo; ++px)
        for (int g = 0; g < G; ++g) {
            float *row = om + px * P + (size_t)g * 3 * K;
            for (int kk = 0; kk < K; ++kk) {
                row[2 * kk] = awkward((float)W);
                row[2 * kk + 1] = awkward((float)H);
                row[2 * K + kk] = uniform(-2.0f, 2.0f);
            }
        }
    float scale = (rnd() % 3) ? 1.0f : 0.5f;
    ++cases;
    if (dcnv4o_forward_ex(v, om, out, N, H, W, k, k, stride, stride, pad, pad, dil, dil, G, Cg, scale, rc, P, sm,
                          1) != K)
        exit(2);
    check_finite(out, no, "conv out");
    ++cases;
    if (dcnv4o_backward_ex(v, om, go, gv, gom, N, H, W, k, k, stride, stride, pad, pad, dil, dil, G, Cg, scale, rc,
                           P, sm, 1) != K)
        exit(2);
    check_finite(gv, nv, "conv grad_value");
    check_finite(gom, nom, "conv grad_offset_mask");
    free(v), free(om), free(go), free(out), free(gv), free(gom);
}

static void fda_case(int N, int L, int Q, int M, int D, int K)
{
    int shapes[8];
    int S = 0;
    for (int l = 0; l < L; ++l) {
        shapes[2 * l] = 1 + (int)(rnd() % 9);
        shapes[2 * l + 1] = 1 + (int)(rnd() % 9);
        S += shapes[2 * l] * shapes[2 * l + 1];
    }
    int P = (3 * L * K + 7) / 8 * 8;
    size_t nv = (size_t)N * S * M * D, nl = (size_t)N * Q * M * P, no = (size_t)N * Q * M * D;
    float *v = malloc(nv * sizeof *v), *loc = malloc(nl * sizeof *loc), *go = malloc(no * sizeof *go);
    double *out = malloc(no * sizeof *out), *gv = malloc(nv * sizeof *gv), *gl = malloc(nl * sizeof *gl);
    for (size_t i = 0; i < nv; ++i)
        v[i] = uniform(-1.0f, 1.0f);
    for (size_t i = 0; i < no; ++i)
        go[i] = uniform(-1.0f, 1.0f);
    for (size_t r = 0; r < (size_t)N * Q * M; ++r) {
        float *row = loc + r * P;
        for (int i = 0; i < L * K; ++i) {
            /* normalised locations: the awkward values scaled to [0, 1] */
            row[2 * i] = awkward(1.0f);
            row[2 * i + 1] = awkward(1.0f);
            row[2 * L * K + i] = uniform(-3.0f, 3.0f);
        }
    }
    ++cases;
    if (fdao_forward(v, shapes, L, loc, out, N, S, Q, M, D, K, P, 1) != 0)
        exit(2);
    check_finite(out, no, "fda out");
    ++cases;
    if (fdao_backward(v, shapes, L, loc, go, gv, gl, N, S, Q, M, D, K, P, 1) != 0)
        exit(2);
    check_finite(gv, nv, "fda grad_value");
    check_finite(gl, nl, "fda grad_loc_attn");
    free(v), free(loc), free(go), free(out), free(gv), free(gl);
}

int main(void)
{
    for (int i = 0; i < 2000; ++i) {
        int k = (int)(rnd() % 3) * 2 + 1;
        conv_case(1 + (int)(rnd() % 2), 1 + (int)(rnd() % 12), 1 + (int)(rnd() % 12), k, 1 + (int)(rnd() % 2),
                  (int)(rnd() % 3), 1 + (int)(rnd() % 2), 1 + (int)(rnd() % 3), 1 + (int)(rnd() % 4),
                  k > 1 && rnd() % 3 == 0, rnd() % 3 == 0);
    }
    for (int i = 0; i < 1000; ++i)
        fda_case(1 + (int)(rnd() % 2), 1 + (int)(rnd() % 4), 1 + (int)(rnd() % 20), 1 + (int)(rnd() % 3),
                 1 + (int)(rnd() % 8), 1 + (int)(rnd() % 4));
    printf("ok %ld\n", cases);
    return 0;
}
