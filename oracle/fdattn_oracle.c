/*
 * Flash deformable attention (multi-scale deformable attention) -- CPU ORACLE.
 *
 * TEST INFRASTRUCTURE ONLY.  Nothing in the product library links, loads or
 * calls this file; only the test suite, the smoke check and the CPU baseline
 * of the benchmark do.  It shares no source with the HIP path.
 *
 * The pages name this operator only: the codewithpapers record of
 * "Efficient Deformable ConvNets" (arXiv 2401.06197) lists the official
 * repository's DCNv4_op/DCNv4/functions/flash_deform_attn_func.py among its
 * code entries, and the blog "DCNv4架构解析" (section "与其他可变形卷积对比")
 * compares DCNv4 with deformable attention.  Its arithmetic is therefore
 * taken from the published definition of multi-scale deformable attention
 * (Zhu et al., "Deformable DETR", ICLR 2021, equation 3), with the input
 * conventions below:
 *
 *   out[n,q,m,:] = sum_{l<L} sum_{k<K} a[n,q,m,l,k] *
 *                  x_l^m( u[n,q,m,l,k] * W_l - 1/2 , v[n,q,m,l,k] * H_l - 1/2 )
 *
 *   - x_l^m(x, y): bilinear sample of the D channels of head m from level
 *     l's H_l x W_l map at column x, row y, zero outside the map.
 *   - (u, v) in [0, 1]: normalised sampling location (u along the width);
 *     pixel (r, c) of level l has its centre at ((c + 1/2) / W_l,
 *     (r + 1/2) / H_l).
 *   - a = softmax over the L*K attention logits of (n, q, m).
 *
 * Readings taken where the pages are silent (each also listed in the design
 * notes of the repository):
 *   F-layout  value (N, S, M, D), S = sum_l H_l*W_l, level l's map in rows
 *             [start_l, start_l + H_l*W_l), start_l = sum_{l'<l} H_l'*W_l',
 *             row-major (r, c).  loc_attn (N, Q, M, P): entries
 *             [2(lK+k), 2(lK+k)+1] = (u, v) of point (l, k), entries
 *             [2LK + lK + k] = its logit, [3LK, P) padding (never read).
 *             Locations and logits in one tensor mirror the merged
 *             offset/mask tensor of DCNv4 (walkthrough section 2.2); the
 *             softmax inside the operator is the "flash" form.
 *   F-coord   x = fmaf(u, (float)W_l, -0.5f), y = fmaf(v, (float)H_l, -0.5f)
 *             in fp32 with one rounding.
 *   F-bound   zero padding: a corner outside [0,H_l) x [0,W_l) contributes 0;
 *             a sample is skipped (every corner outside) unless
 *             -1 <= y < H_l and -1 <= x < W_l; NaN locations are skipped.
 *   F-deriv   at integer coordinates the derivative is the right derivative
 *             (that of the cell chosen by floor).
 *   F-softmax the softmax runs over all L*K points of (n, q, m), live or not,
 *             in double, with the maximum subtracted; its gradient is the
 *             softmax Jacobian: dL/dz_i = a_i (dL/da_i - sum_j a_j dL/da_j).
 *   F-grad    backward overwrites its outputs; padding entries of
 *             grad_loc_attn are 0.
 *
 * Weights are formed in fp32 exactly as written below (one rounding per
 * product); everything after the weights is accumulated in double.
 *
 * Pins (tests that tie this oracle to something other than itself): torch
 * grid_sample (bilinear, zeros, align_corners=False) and softmax with
 * autograd in float64, exact gathers at pixel centres, constant and affine
 * maps, shift invariance of the logits, the adjoint identity for
 * grad_value, and finite differences for the locations and logits.
 */
#include <math.h>
#include <stdint.h>
#include <stdlib.h>
#include <string.h>

#ifdef _OPENMP
#include <omp.h>
#endif

#define FDAO_MAX_LEVELS 64

typedef struct {
    int live;
    int r0, c0;      /* top-left corner (row, column) */
    float ly, lx;    /* fractional parts */
    float hy, hx;    /* 1 - ly, 1 - lx */
    float wt[4];     /* weights of (r0,c0), (r0,c0+1), (r0+1,c0), (r0+1,c0+1) */
} fdao_footprint;

static fdao_footprint fdao_bilinear(float y, float x, int H, int W)
{
    fdao_footprint f;
    memset(&f, 0, sizeof f);
    if (!(y >= -1.0f && y < (float)H && x >= -1.0f && x < (float)W))
        return f; /* also false for NaN */
    float fy = floorf(y);
    float fx = floorf(x);
    f.live = 1;
    f.r0 = (int)fy;
    f.c0 = (int)fx;
    f.ly = y - fy;
    f.lx = x - fx;
    f.hy = 1.0f - f.ly;
    f.hx = 1.0f - f.lx;
    f.wt[0] = f.hy * f.hx;
    f.wt[1] = f.hy * f.lx;
    f.wt[2] = f.ly * f.hx;
    f.wt[3] = f.ly * f.lx;
    return f;
}

/* Softmax of n logits in double (F-softmax). */
static void fdao_softmax(const float *z, int n, double *a)
{
    double mx = (double)z[0];
    for (int i = 1; i < n; ++i)
        if ((double)z[i] > mx)
            mx = (double)z[i];
    double sum = 0.0;
    for (int i = 0; i < n; ++i) {
        a[i] = exp((double)z[i] - mx);
        sum += a[i];
    }
    for (int i = 0; i < n; ++i)
        a[i] /= sum;
}

/* Checks the level shapes; fills start[]; returns 0 or -1. */
static int fdao_levels(const int *shapes, int L, int S, long *start)
{
    if (L < 1 || L > FDAO_MAX_LEVELS)
        return -1;
    long s = 0;
    for (int l = 0; l < L; ++l) {
        if (shapes[2 * l] < 1 || shapes[2 * l + 1] < 1)
            return -1;
        start[l] = s;
        s += (long)shapes[2 * l] * shapes[2 * l + 1];
    }
    return s == (long)S ? 0 : -1;
}

/* Value of head m, channel d at pixel (r, c) of level l (zero outside). */
static double fdao_x(const float *value, int n, long start, int r, int c, int H, int W,
                     int S, int M, int D, int m, int d)
{
    if (r < 0 || r >= H || c < 0 || c >= W)
        return 0.0;
    long s = start + (long)r * W + c;
    return (double)value[(((size_t)n * S + s) * M + m) * D + d];
}

/*
 * Forward.  value (N,S,M,D) fp32; shapes (L,2) = (H_l, W_l); loc_attn
 * (N,Q,M,P) fp32; out (N,Q,M,D) double.  nthreads <= 0: OpenMP default.
 * Returns 0, or -1 on bad arguments.
 */
int fdao_forward(const float *value, const int *shapes, int L, const float *loc_attn, double *out,
                 int N, int S, int Q, int M, int D, int K, int P, int nthreads)
{
    long start[FDAO_MAX_LEVELS];
    if (fdao_levels(shapes, L, S, start) != 0 || K < 1 || P < 3 * L * K || M < 1 || D < 1)
        return -1;
    int LK = L * K;
    long units = (long)N * Q * M;
#ifdef _OPENMP
    int nt = nthreads > 0 ? nthreads : omp_get_max_threads();
#pragma omp parallel for schedule(dynamic, 256) num_threads(nt)
#endif
    for (long u = 0; u < units; ++u) {
        int n = (int)(u / ((long)Q * M));
        int m = (int)(u % M);
        const float *row = loc_attn + (size_t)u * P;
        double *y = out + (size_t)u * D;
        double *a = (double *)malloc(sizeof(double) * (size_t)LK);
        fdao_softmax(row + 2 * LK, LK, a);
        for (int d = 0; d < D; ++d)
            y[d] = 0.0;
        for (int l = 0; l < L; ++l) {
            int H = shapes[2 * l], W = shapes[2 * l + 1];
            for (int k = 0; k < K; ++k) {
                int i = l * K + k;
                float x = fmaf(row[2 * i], (float)W, -0.5f);
                float yy = fmaf(row[2 * i + 1], (float)H, -0.5f);
                fdao_footprint f = fdao_bilinear(yy, x, H, W);
                if (!f.live)
                    continue;
                for (int d = 0; d < D; ++d) {
                    double s = (double)f.wt[0] * fdao_x(value, n, start[l], f.r0, f.c0, H, W, S, M, D, m, d)
                             + (double)f.wt[1] * fdao_x(value, n, start[l], f.r0, f.c0 + 1, H, W, S, M, D, m, d)
                             + (double)f.wt[2] * fdao_x(value, n, start[l], f.r0 + 1, f.c0, H, W, S, M, D, m, d)
                             + (double)f.wt[3] * fdao_x(value, n, start[l], f.r0 + 1, f.c0 + 1, H, W, S, M, D, m, d);
                    y[d] += a[i] * s;
                }
            }
        }
        free(a);
    }
    return 0;
}

/*
 * Backward (chain rule of the forward above).  grad_out (N,Q,M,D) fp32.
 * Outputs (overwritten): grad_value (N,S,M,D) double, grad_loc_attn
 * (N,Q,M,P) double with zeros in the padding.
 *
 *   d out_d / d a_i      = s_{i,d}                        (bilinear sample)
 *   d out_d / d u_i      = a_i * W_l * (hy*(v01 - v00) + ly*(v11 - v10))
 *   d out_d / d v_i      = a_i * H_l * (hx*(v10 - v00) + lx*(v11 - v01))
 *   d out_d / d x[corner]= a_i * weight(corner)   (in-map corners only)
 *   d L / d z_i          = a_i * (dL/da_i - sum_j a_j dL/da_j)
 *
 * Parallel over images n (disjoint grad_value slices): deterministic.
 * Returns 0, or -1 on bad arguments.
 */
int fdao_backward(const float *value, const int *shapes, int L, const float *loc_attn,
                  const float *grad_out, double *grad_value, double *grad_loc_attn,
                  int N, int S, int Q, int M, int D, int K, int P, int nthreads)
{
    long start[FDAO_MAX_LEVELS];
    if (fdao_levels(shapes, L, S, start) != 0 || K < 1 || P < 3 * L * K || M < 1 || D < 1)
        return -1;
    int LK = L * K;
    memset(grad_value, 0, sizeof(double) * (size_t)N * S * M * D);
    memset(grad_loc_attn, 0, sizeof(double) * (size_t)N * Q * M * P);
#ifdef _OPENMP
    int nt = nthreads > 0 ? nthreads : omp_get_max_threads();
#pragma omp parallel for schedule(dynamic, 1) num_threads(nt)
#endif
    for (int n = 0; n < N; ++n) {
        double *a = (double *)malloc(sizeof(double) * (size_t)LK);
        double *ga = (double *)malloc(sizeof(double) * (size_t)LK);
        for (int q = 0; q < Q; ++q) {
            for (int m = 0; m < M; ++m) {
                size_t u = ((size_t)n * Q + q) * M + m;
                const float *row = loc_attn + u * P;
                const float *g = grad_out + u * D;
                double *grow = grad_loc_attn + u * P;
                fdao_softmax(row + 2 * LK, LK, a);
                for (int l = 0; l < L; ++l) {
                    int H = shapes[2 * l], W = shapes[2 * l + 1];
                    for (int k = 0; k < K; ++k) {
                        int i = l * K + k;
                        ga[i] = 0.0;
                        float x = fmaf(row[2 * i], (float)W, -0.5f);
                        float yy = fmaf(row[2 * i + 1], (float)H, -0.5f);
                        fdao_footprint f = fdao_bilinear(yy, x, H, W);
                        if (!f.live)
                            continue; /* location gradients stay 0 */
                        int rr[4] = {f.r0, f.r0, f.r0 + 1, f.r0 + 1};
                        int cc[4] = {f.c0, f.c0 + 1, f.c0, f.c0 + 1};
                        double gs = 0.0, gx = 0.0, gy = 0.0;
                        for (int d = 0; d < D; ++d) {
                            double go = (double)g[d];
                            double v[4];
                            for (int c = 0; c < 4; ++c)
                                v[c] = fdao_x(value, n, start[l], rr[c], cc[c], H, W, S, M, D, m, d);
                            double s = (double)f.wt[0] * v[0] + (double)f.wt[1] * v[1]
                                     + (double)f.wt[2] * v[2] + (double)f.wt[3] * v[3];
                            gs += go * s;
                            gx += go * ((double)f.hy * (v[1] - v[0]) + (double)f.ly * (v[3] - v[2]));
                            gy += go * ((double)f.hx * (v[2] - v[0]) + (double)f.lx * (v[3] - v[1]));
                            for (int c = 0; c < 4; ++c) {
                                if (rr[c] < 0 || rr[c] >= H || cc[c] < 0 || cc[c] >= W)
                                    continue;
                                long s_idx = start[l] + (long)rr[c] * W + cc[c];
                                grad_value[(((size_t)n * S + s_idx) * M + m) * D + d] += a[i] * (double)f.wt[c] * go;
                            }
                        }
                        ga[i] = gs;
                        grow[2 * i] = a[i] * (double)W * gx;
                        grow[2 * i + 1] = a[i] * (double)H * gy;
                    }
                }
                double dot = 0.0;
                for (int i = 0; i < LK; ++i)
                    dot += a[i] * ga[i];
                for (int i = 0; i < LK; ++i)
                    grow[2 * LK + i] = a[i] * (ga[i] - dot);
            }
        }
        free(ga);
        free(a);
    }
    return 0;
}
