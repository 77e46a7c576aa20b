/*
 * DCNv4 spatial aggregation -- CPU ORACLE.
 *
 * TEST INFRASTRUCTURE ONLY.  Nothing in the product library links, loads or
 * calls this file; only the test suite, the smoke check and the CPU baseline
 * of the benchmark do.  It shares no source with the HIP path.
 *
 * What it computes (plain definition, double accumulation):
 *
 *   y_g(p0) = sum_{k=1..K} m_gk * x_g(p0 + p_k + offset_scale * dp_gk)
 *   y       = concat_g y_g  along the channel (last) axis
 *
 *   - The aggregation formula and the per-group slicing x_g, y_g with
 *     C' = C / G channels: "Efficient Deformable ConvNets" as summarised in the
 *     CSDN walkthrough "DCNv4论文解析", section 1.2 (DCNv3 recap equation).
 *   - No softmax over K: m is an unnormalised, signed scalar (same walkthrough,
 *     section 2.1, "增强动态特性").  The _ex entry points also offer the
 *     DCNv3 form that section 2.1 contrasts it with (the recap equation of
 *     section 1.2 with m normalised by a softmax over the K points of each
 *     pixel and group): with softmax != 0, m_gk is replaced by
 *     p_gk = exp(m_gk) / sum_j exp(m_gj), computed in double.
 *   - The scalar offset_scale, stride, pad, dilation and remove_center
 *     arguments: the dcnv4_cuda_forward / DCNv4Function.forward argument lists
 *     quoted in the blog "DCNv4架构解析", sections "内存访问优化策略" and
 *     "计算图优化".
 *   - x_g(p) at a fractional p is a bilinear sample ("x4 for bilinear
 *     interpolation per sampling point", walkthrough section 2.2).
 *   - The fused offset/mask tensor (one merged linear, last dim padded to a
 *     multiple of 8): walkthrough section 2.2 (micro-design) and the blog's
 *     "内存访问优化策略" (padded_offset_dim divisible by 8).
 *
 * Readings taken where the pages are silent (each also listed in the design
 * notes of the repository):
 *   R-layout  offset_mask row of a pixel = for g in 0..G-1:
 *             [dx_0, dy_0, dx_1, dy_1, ..., dx_{K-1}, dy_{K-1}, m_0 .. m_{K-1}],
 *             then padding up to P channels (never read).
 *   R-order   grid point k enumerates i over kernel_w (x) outer and j over
 *             kernel_h (y) inner, skipping the centre when remove_center.
 *   R-coord   loc_w = fmaf(offset_scale, dx, (float)(wo*stride_w - pad_w + i*dil_w))
 *             loc_h = fmaf(offset_scale, dy, (float)(ho*stride_h - pad_h + j*dil_h))
 *             in fp32 with a single rounding; integer (h, w) samples x[h][w]
 *             exactly (no half-pixel shift).
 *   R-bound   zero-extended image: each bilinear corner outside [0,H)x[0,W)
 *             contributes 0.  A sample is skipped (all four corners outside)
 *             unless -1 <= loc < size on both axes; NaN locations are skipped.
 *   R-deriv   at integer coordinates the derivative is the right derivative
 *             (that of the cell chosen by floor).
 *   R-grad    backward overwrites its outputs; padding entries of
 *             grad_offset_mask are 0.
 *
 * Weights are formed in fp32 exactly as written below (one rounding per
 * product); everything after the weights is accumulated in double.
 *
 *   R-softmax the softmax runs over all K points of a (pixel, group), live or
 *             not (a point outside the image keeps its share of the weight
 *             and samples zeros); its gradient is the softmax Jacobian:
 *             dL/dm_k = p_k * (dL/dp_k - sum_j p_j * dL/dp_j).
 *
 * Pins (tests that tie this oracle to something other than itself): identity
 * and stride-2 subsampling with a one-hot centre mask, grouped depthwise
 * convolution for zero offsets, exact gathers for integer offsets, the affine
 * image closed form, torch grid_sample reduction, linearity, adjoint
 * identities for grad_value / grad_mask, finite differences for
 * grad_offset, and a brute-force zero-padded formulation on tiny inputs.
 */
#include <math.h>
#include <stdint.h>
#include <stdlib.h>
#include <string.h>

#ifdef _OPENMP
#include <omp.h>
#endif

#define ORACLE_MAX_K 1024

/* Output spatial size: standard convolution geometry. */
int dcnv4o_output_size(int in, int kernel, int stride, int pad, int dil)
{
    int span = dil * (kernel - 1) + 1;
    return (in + 2 * pad - span) / stride + 1;
}

/* Grid point list (R-order).  Returns K; fills gi (x index) and gj (y index). */
int dcnv4o_grid(int kernel_h, int kernel_w, int remove_center, int *gi, int *gj)
{
    int K = 0;
    for (int i = 0; i < kernel_w; ++i) {
        for (int j = 0; j < kernel_h; ++j) {
            if (remove_center && i == (kernel_w - 1) / 2 && j == (kernel_h - 1) / 2)
                continue;
            gi[K] = i;
            gj[K] = j;
            ++K;
        }
    }
    return K;
}

/* Bilinear footprint of one sample: four corners and their fp32 weights. */
typedef struct {
    int live;       /* 0: sample skipped, contributes nothing */
    int h0, w0;     /* top-left corner */
    float lh, lw;   /* fractional parts */
    float hh, hw;   /* 1 - lh, 1 - lw */
    float wt[4];    /* weights of (h0,w0), (h0,w0+1), (h0+1,w0), (h0+1,w0+1) */
} footprint;

static footprint bilinear_footprint(float loc_h, float loc_w, int H, int W)
{
    footprint f;
    memset(&f, 0, sizeof f);
    if (!(loc_h >= -1.0f && loc_h < (float)H && loc_w >= -1.0f && loc_w < (float)W))
        return f; /* also false for NaN */
    float fh = floorf(loc_h);
    float fw = floorf(loc_w);
    f.live = 1;
    f.h0 = (int)fh;
    f.w0 = (int)fw;
    f.lh = loc_h - fh;
    f.lw = loc_w - fw;
    f.hh = 1.0f - f.lh;
    f.hw = 1.0f - f.lw;
    f.wt[0] = f.hh * f.hw;
    f.wt[1] = f.hh * f.lw;
    f.wt[2] = f.lh * f.hw;
    f.wt[3] = f.lh * f.lw;
    return f;
}

/* Softmax of the K masks of one (pixel, group) in double (R-softmax). */
static void softmax_masks(const float *m, int K, double *p)
{
    double mx = (double)m[0];
    for (int k = 1; k < K; ++k)
        if ((double)m[k] > mx)
            mx = (double)m[k];
    double sum = 0.0;
    for (int k = 0; k < K; ++k) {
        p[k] = exp((double)m[k] - mx);
        sum += p[k];
    }
    for (int k = 0; k < K; ++k)
        p[k] /= sum;
}

/* Value of the zero-extended image x[n][r][c][ch] (channel-last). */
static double xval(const float *value, int n, int r, int c, int ch, int H, int W, int C)
{
    if (r < 0 || r >= H || c < 0 || c >= W)
        return 0.0;
    return (double)value[(((size_t)n * H + r) * W + c) * C + ch];
}

/*
 * Forward.  value: (N,H,W,G*Cg) fp32; offset_mask: (N,Ho,Wo,P) fp32;
 * out: (N,Ho,Wo,G*Cg) double.  Inputs in other storage types are upcast
 * exactly to fp32 by the caller.  nthreads <= 0 means the OpenMP default.
 * Returns K, or -1 on bad geometry.
 */
int dcnv4o_forward_ex(const float *value, const float *offset_mask, double *out,
                      int N, int H, int W, int kernel_h, int kernel_w,
                      int stride_h, int stride_w, int pad_h, int pad_w,
                      int dil_h, int dil_w, int G, int Cg, float offset_scale,
                      int remove_center, int P, int softmax, int nthreads)
{
    int gi[ORACLE_MAX_K], gj[ORACLE_MAX_K];
    if ((size_t)kernel_h * kernel_w > ORACLE_MAX_K)
        return -1;
    int K = dcnv4o_grid(kernel_h, kernel_w, remove_center, gi, gj);
    int Ho = dcnv4o_output_size(H, kernel_h, stride_h, pad_h, dil_h);
    int Wo = dcnv4o_output_size(W, kernel_w, stride_w, pad_w, dil_w);
    int C = G * Cg;
    if (Ho <= 0 || Wo <= 0 || P < 3 * G * K)
        return -1;
    long rows = (long)N * Ho;
#ifdef _OPENMP
    int nt = nthreads > 0 ? nthreads : omp_get_max_threads();
#pragma omp parallel for schedule(dynamic, 1) num_threads(nt)
#endif
    for (long row = 0; row < rows; ++row) {
        int n = (int)(row / Ho);
        int ho = (int)(row % Ho);
        double *acc = (double *)malloc(sizeof(double) * (size_t)(Cg > 0 ? Cg : 1));
        double *pk = (double *)malloc(sizeof(double) * (size_t)K);
        for (int wo = 0; wo < Wo; ++wo) {
            const float *om = offset_mask + (((size_t)n * Ho + ho) * Wo + wo) * P;
            double *y = out + (((size_t)n * Ho + ho) * Wo + wo) * C;
            for (int g = 0; g < G; ++g) {
                const float *omg = om + (size_t)g * 3 * K;
                for (int c = 0; c < Cg; ++c)
                    acc[c] = 0.0;
                if (softmax)
                    softmax_masks(omg + 2 * K, K, pk);
                for (int k = 0; k < K; ++k) {
                    float dx = omg[2 * k];
                    float dy = omg[2 * k + 1];
                    double m = softmax ? pk[k] : (double)omg[2 * K + k];
                    float loc_w = fmaf(offset_scale, dx, (float)(wo * stride_w - pad_w + gi[k] * dil_w));
                    float loc_h = fmaf(offset_scale, dy, (float)(ho * stride_h - pad_h + gj[k] * dil_h));
                    footprint f = bilinear_footprint(loc_h, loc_w, H, W);
                    if (!f.live)
                        continue;
                    for (int c = 0; c < Cg; ++c) {
                        int ch = g * Cg + c;
                        double s = (double)f.wt[0] * xval(value, n, f.h0, f.w0, ch, H, W, C)
                                 + (double)f.wt[1] * xval(value, n, f.h0, f.w0 + 1, ch, H, W, C)
                                 + (double)f.wt[2] * xval(value, n, f.h0 + 1, f.w0, ch, H, W, C)
                                 + (double)f.wt[3] * xval(value, n, f.h0 + 1, f.w0 + 1, ch, H, W, C);
                        acc[c] += m * s;
                    }
                }
                for (int c = 0; c < Cg; ++c)
                    y[g * Cg + c] = acc[c];
            }
        }
        free(pk);
        free(acc);
    }
    return K;
}

int dcnv4o_forward(const float *value, const float *offset_mask, double *out,
                   int N, int H, int W, int kernel_h, int kernel_w,
                   int stride_h, int stride_w, int pad_h, int pad_w,
                   int dil_h, int dil_w, int G, int Cg, float offset_scale,
                   int remove_center, int P, int nthreads)
{
    return dcnv4o_forward_ex(value, offset_mask, out, N, H, W, kernel_h, kernel_w, stride_h, stride_w,
                             pad_h, pad_w, dil_h, dil_w, G, Cg, offset_scale, remove_center, P, 0, nthreads);
}

/*
 * Backward (chain rule of the forward above; the pages describe no backward
 * algorithm).  grad_out: (N,Ho,Wo,G*Cg) fp32.  Outputs (overwritten):
 * grad_value (N,H,W,G*Cg) double; grad_offset_mask (N,Ho,Wo,P) double with
 * the same channel layout as offset_mask and zeros in the padding.
 *
 *   d y_c / d m_gk     = s_c                      (the bilinear sample)
 *   d y_c / d loc_w    = m * (hh*(v01 - v00) + lh*(v11 - v10))
 *   d y_c / d loc_h    = m * (hw*(v10 - v00) + lw*(v11 - v01))
 *   d loc / d dp       = offset_scale
 *   d y_c / d x[corner]= m * weight(corner)   (in-bounds corners only)
 *
 * Parallel over images n: grad_value slices of different images are
 * disjoint, so each image is accumulated serially and the result is
 * deterministic.  Returns K, or -1 on bad geometry.
 */
int dcnv4o_backward_ex(const float *value, const float *offset_mask, const float *grad_out,
                       double *grad_value, double *grad_offset_mask,
                       int N, int H, int W, int kernel_h, int kernel_w,
                       int stride_h, int stride_w, int pad_h, int pad_w,
                       int dil_h, int dil_w, int G, int Cg, float offset_scale,
                       int remove_center, int P, int softmax, int nthreads)
{
    int gi[ORACLE_MAX_K], gj[ORACLE_MAX_K];
    if ((size_t)kernel_h * kernel_w > ORACLE_MAX_K)
        return -1;
    int K = dcnv4o_grid(kernel_h, kernel_w, remove_center, gi, gj);
    int Ho = dcnv4o_output_size(H, kernel_h, stride_h, pad_h, dil_h);
    int Wo = dcnv4o_output_size(W, kernel_w, stride_w, pad_w, dil_w);
    int C = G * Cg;
    if (Ho <= 0 || Wo <= 0 || P < 3 * G * K)
        return -1;
    memset(grad_value, 0, sizeof(double) * (size_t)N * H * W * C);
    memset(grad_offset_mask, 0, sizeof(double) * (size_t)N * Ho * Wo * P);
#ifdef _OPENMP
    int nt = nthreads > 0 ? nthreads : omp_get_max_threads();
#pragma omp parallel for schedule(dynamic, 1) num_threads(nt)
#endif
    for (int n = 0; n < N; ++n) {
        double *gv = grad_value + (size_t)n * H * W * C;
        double *pk = (double *)malloc(sizeof(double) * (size_t)K);
        for (int ho = 0; ho < Ho; ++ho) {
            for (int wo = 0; wo < Wo; ++wo) {
                size_t pix = ((size_t)n * Ho + ho) * Wo + wo;
                const float *om = offset_mask + pix * P;
                const float *gy = grad_out + pix * C;
                double *gom = grad_offset_mask + pix * P;
                for (int g = 0; g < G; ++g) {
                    const float *omg = om + (size_t)g * 3 * K;
                    double *gomg = gom + (size_t)g * 3 * K;
                    if (softmax)
                        softmax_masks(omg + 2 * K, K, pk);
                    for (int k = 0; k < K; ++k) {
                        float dx = omg[2 * k];
                        float dy = omg[2 * k + 1];
                        double m = softmax ? pk[k] : (double)omg[2 * K + k];
                        float loc_w = fmaf(offset_scale, dx, (float)(wo * stride_w - pad_w + gi[k] * dil_w));
                        float loc_h = fmaf(offset_scale, dy, (float)(ho * stride_h - pad_h + gj[k] * dil_h));
                        footprint f = bilinear_footprint(loc_h, loc_w, H, W);
                        if (!f.live)
                            continue; /* gradients stay 0 */
                        int rr[4] = {f.h0, f.h0, f.h0 + 1, f.h0 + 1};
                        int cc[4] = {f.w0, f.w0 + 1, f.w0, f.w0 + 1};
                        double gm = 0.0, gw = 0.0, gh = 0.0;
                        for (int c = 0; c < Cg; ++c) {
                            int ch = g * Cg + c;
                            double go = (double)gy[ch];
                            double v[4];
                            for (int q = 0; q < 4; ++q)
                                v[q] = xval(value, n, rr[q], cc[q], ch, H, W, C);
                            double s = (double)f.wt[0] * v[0] + (double)f.wt[1] * v[1]
                                     + (double)f.wt[2] * v[2] + (double)f.wt[3] * v[3];
                            gm += go * s;
                            gw += go * ((double)f.hh * (v[1] - v[0]) + (double)f.lh * (v[3] - v[2]));
                            gh += go * ((double)f.hw * (v[2] - v[0]) + (double)f.lw * (v[3] - v[1]));
                            for (int q = 0; q < 4; ++q) {
                                if (rr[q] < 0 || rr[q] >= H || cc[q] < 0 || cc[q] >= W)
                                    continue;
                                gv[((size_t)rr[q] * W + cc[q]) * C + ch] += m * (double)f.wt[q] * go;
                            }
                        }
                        gomg[2 * k] = (double)offset_scale * m * gw;
                        gomg[2 * k + 1] = (double)offset_scale * m * gh;
                        gomg[2 * K + k] = gm;
                    }
                    if (softmax) {
                        /* dL/dm_k = p_k * (dL/dp_k - sum_j p_j dL/dp_j) (R-softmax) */
                        double s = 0.0;
                        for (int k = 0; k < K; ++k)
                            s += pk[k] * gomg[2 * K + k];
                        for (int k = 0; k < K; ++k)
                            gomg[2 * K + k] = pk[k] * (gomg[2 * K + k] - s);
                    }
                }
            }
        }
        free(pk);
    }
    return K;
}

int dcnv4o_backward(const float *value, const float *offset_mask, const float *grad_out,
                    double *grad_value, double *grad_offset_mask,
                    int N, int H, int W, int kernel_h, int kernel_w,
                    int stride_h, int stride_w, int pad_h, int pad_w,
                    int dil_h, int dil_w, int G, int Cg, float offset_scale,
                    int remove_center, int P, int nthreads)
{
    return dcnv4o_backward_ex(value, offset_mask, grad_out, grad_value, grad_offset_mask, N, H, W, kernel_h,
                              kernel_w, stride_h, stride_w, pad_h, pad_w, dil_h, dil_w, G, Cg, offset_scale,
                              remove_center, P, 0, nthreads);
}
