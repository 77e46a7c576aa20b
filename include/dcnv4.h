/*
 * dcnv4.h -- C ABI of the MI355X (gfx950) DCNv4 spatial-aggregation library
 * (libdcnv4.so).
 *
 * The operation (forward):
 *
 *   y_g(p0) = sum_{k=0..K-1} m_gk * x_g(p0 + p_k + offset_scale * dp_gk)
 *   y       = concat over groups g of y_g along the channel axis
 *
 * for every output pixel p0 and group g, where x_g is the g-th slice of C'
 * (= group_channels) channels of the input, p_k is the k-th point of the
 * regular kernel_h x kernel_w grid (dilated, strided, padded as in a regular
 * convolution), dp_gk = (dx, dy) is a learned fractional offset and m_gk an
 * unnormalised, signed modulation scalar (no softmax over k).  x_g at a
 * fractional location is a bilinear sample of the zero-extended image.
 * Sources: "Efficient Deformable ConvNets: Rethinking Dynamic and Sparse
 * Operator for Vision Applications" as summarised by the CSDN walkthrough
 * "DCNv4论文解析", section 1.2 (DCNv3 recap equation), section 2.1 (softmax
 * removed: m is unbounded) and section 2.2 (bilinear sampling; D' channels of
 * a group share offsets and coefficients; channel-last layout; fused
 * offset/mask tensor); the argument list of dcnv4_cuda_forward quoted in the
 * blog "DCNv4架构解析", section "内存访问优化策略" (kernel, stride, pad,
 * dilation, group, group_channels, offset_scale, remove_center; offset row
 * padded to a multiple of 8).
 *
 * Conventions fixed by this library (where the pages are silent):
 *   - value      : (N, H, W, G*C') channel-last, dense.
 *   - offset_mask: (N, Ho, Wo, P) channel-last, dense; per pixel, for each
 *                  group g the 3K entries [g*3K, g*3K+3K) hold
 *                  dx_0, dy_0, dx_1, dy_1, ..., dx_{K-1}, dy_{K-1}, m_0..m_{K-1};
 *                  entries [3GK, P) are padding and never read.
 *   - grid order : k enumerates i = 0..kernel_w-1 (x, outer) and
 *                  j = 0..kernel_h-1 (y, inner), skipping the centre
 *                  ((kernel_w-1)/2, (kernel_h-1)/2) when remove_center.
 *   - coordinate : loc_w = fmaf(offset_scale, dx, wo*stride_w - pad_w + i*dilation_w)
 *                  loc_h = fmaf(offset_scale, dy, ho*stride_h - pad_h + j*dilation_h)
 *                  in fp32 (one rounding); pixel (h, w) samples x[h][w] exactly.
 *   - border     : a bilinear corner outside [0,H)x[0,W) contributes 0; a
 *                  sample with loc outside [-1,H)x[-1,W) (or NaN) contributes
 *                  nothing.  value and the masks must be finite.
 *   - output     : (N, Ho, Wo, G*C') channel-last, overwritten.
 *   - arithmetic : fp32 coordinates, weights and accumulation; outputs are
 *                  rounded to nearest-even into the storage dtype.
 *
 * Ownership and execution, all entry points:
 *   - The caller allocates every buffer (device memory for tensors), dense,
 *     with 16-byte aligned base pointers.  The library allocates nothing,
 *     frees nothing and keeps no pointer after returning.  (One static
 *     device array exists, the scratch of flash_deform_attn_backward_noalloc
 *     in flash_deform_attn.h; no DCNv4 entry point uses it.)
 *   - Work is enqueued on `stream` (a hipStream_t passed as void*; NULL is
 *     the null stream) and the call returns without waiting; results are
 *     valid once the stream has completed the work.
 *   - Outputs must not overlap inputs or each other.
 *   - Reentrant.  Process state: a per-thread copy of the last HIP error
 *     message; a record of the kernels whose dynamic-LDS limit has been
 *     raised (hipFuncSetAttribute, once per kernel and device, under a
 *     lock); and two caches of tile plans (forward, backward), each of up
 *     to 64 geometries, keyed by the call's scalar arguments (not by
 *     pointers), filled on first use and shared by all threads under a
 *     lock.  None of it holds device memory or caller pointers.
 *
 * Errors: every entry point returns DCNV4_OK (0) or a negative status.  All
 * argument checks run before any HIP call, so a rejected call has no side
 * effects.  N == 0 is a valid no-op (pointers may then be NULL).
 */
#ifndef DCNV4_H
#define DCNV4_H

#if defined(__GNUC__)
#define DCNV4_API __attribute__((visibility("default")))
#else
#define DCNV4_API
#endif

#ifdef __cplusplus
extern "C" {
#endif

#define DCNV4_ABI_VERSION 3

enum dcnv4_status {
    DCNV4_OK = 0,
    DCNV4_ERR_NULL = -1,        /* a required pointer is NULL */
    DCNV4_ERR_SHAPE = -2,       /* non-positive size, or empty output */
    DCNV4_ERR_PARAM = -3,       /* bad stride/pad/dilation/group/om_channels/remove_center, overlap */
    DCNV4_ERR_DTYPE = -4,       /* dtype not one of enum dcnv4_dtype */
    DCNV4_ERR_ALIGN = -5,       /* a base pointer is not 16-byte aligned */
    DCNV4_ERR_UNSUPPORTED = -6, /* valid but not implemented (see each call) */
    DCNV4_ERR_OVERFLOW = -7,    /* a size exceeds the library's index range */
    DCNV4_ERR_HIP = -8          /* the HIP runtime reported an error */
};

enum dcnv4_dtype {
    DCNV4_FP32 = 0,
    DCNV4_FP16 = 1, /* IEEE binary16 storage, fp32 arithmetic */
    DCNV4_BF16 = 2  /* bfloat16 storage, fp32 arithmetic */
};

/* DCNV4_ABI_VERSION of the built library. */
DCNV4_API int dcnv4_abi_version(void);

/* Static text for a status code (never NULL). */
DCNV4_API const char *dcnv4_status_string(int status);

/* Text of the last HIP error seen by this thread inside the library ("" if
 * none).  Valid until the next library call on the same thread. */
DCNV4_API const char *dcnv4_last_hip_error(void);

/*
 * Output size of the sampling grid, as for a regular convolution (the
 * sampling grid p0 + p_k is that of a regular convolution when the offsets
 * are zero: walkthrough "DCNv4论文解析", section 1.2):
 *   Ho = floor((H + 2*pad_h - (dilation_h*(kernel_h-1) + 1)) / stride_h) + 1
 * and likewise Wo.  Writes *Ho, *Wo.  Errors: NULL, PARAM (kernel, stride,
 * dilation < 1 or pad < 0), SHAPE (H, W < 1 or Ho, Wo < 1).
 */
DCNV4_API int dcnv4_output_size(int H, int W, int kernel_h, int kernel_w, int stride_h, int stride_w,
                      int pad_h, int pad_w, int dilation_h, int dilation_w, int *Ho, int *Wo);

/*
 * Smallest valid om_channels: 3*group*K rounded up to a multiple of 8, with
 * K = kernel_h*kernel_w - (remove_center ? 1 : 0) (walkthrough section 2.2:
 * offsets (G, K*2) and weights (G, K) merged into one tensor; blog section
 * "内存访问优化策略": padded to a multiple of 8).  Returns a positive value,
 * or DCNV4_ERR_PARAM.
 */
DCNV4_API int dcnv4_om_channels(int group, int kernel_h, int kernel_w, int remove_center);

/*
 * Forward spatial aggregation (the operation above).
 *
 *   value        (N, H, W, group*group_channels)  dtype, read
 *   offset_mask  (N, Ho, Wo, om_channels)         dtype, read
 *   output       (N, Ho, Wo, group*group_channels) dtype, written
 *
 * dtype: enum dcnv4_dtype, the same for all three tensors.
 * remove_center: 0 or 1; 1 drops the grid centre (needs odd kernel sizes,
 * kernel_h*kernel_w > 1).  om_channels: >= 3*group*K and a multiple of 8.
 * Errors: NULL, SHAPE, PARAM, DTYPE, ALIGN, OVERFLOW (one image of any
 * tensor exceeds 2^31 bytes, or N*Ho*Wo*group exceeds 2^31),
 * UNSUPPORTED (group_channels * sizeof(dtype) not a multiple of 16 bytes, or
 * K*group too large for the on-chip staging), HIP.
 */
DCNV4_API int dcnv4_forward(const void *value, const void *offset_mask, void *output,
                  int N, int H, int W, int kernel_h, int kernel_w,
                  int stride_h, int stride_w, int pad_h, int pad_w,
                  int dilation_h, int dilation_w, int group, int group_channels,
                  float offset_scale, int remove_center, int om_channels,
                  int dtype, void *stream);

/*
 * Backward of dcnv4_forward (chain rule of the operation above; the pages
 * give no backward algorithm):
 *
 *   grad_value[x corner]     = sum over samples of m * bilinear weight * grad_output
 *   grad_offset_mask dx, dy  = offset_scale * m * sum_c grad_output_c * d sample_c / d loc
 *                              (right derivative at integer coordinates)
 *   grad_offset_mask m       = sum_c grad_output_c * sample_c
 *
 *   value, offset_mask       as for dcnv4_forward, read
 *   grad_output      (N, Ho, Wo, group*group_channels), read
 *   grad_value       (N, H, W, group*group_channels) fp32 for every dtype,
 *                    written (overwritten, not accumulated)
 *   grad_offset_mask (N, Ho, Wo, om_channels), written; padding entries 0
 *
 * dtype: of value, offset_mask, grad_output and grad_offset_mask (grad_value
 * is always fp32, so that the many contributions to one element are summed
 * and rounded once; a caller that wants it in 16 bits rounds it once).  fp32
 * for every geometry dcnv4_forward accepts; fp16 and bf16 (fp32 arithmetic,
 * grad_offset_mask rounded to nearest-even into the storage dtype) when the
 * LDS-tiled kernels cover the geometry: group_channels in {8, 16, 32} and
 * K <= 25, otherwise DCNV4_ERR_UNSUPPORTED.
 * grad_offset_mask is deterministic.  grad_value is summed in an order that
 * depends on thread timing (an on-chip counting sort of the samples, and
 * device atomics for samples that land more than a few pixels from their
 * grid position), so its last bits may differ from run to run.
 * Errors: as dcnv4_forward.
 */
DCNV4_API int dcnv4_backward(const void *value, const void *offset_mask, const void *grad_output,
                   void *grad_value, void *grad_offset_mask,
                   int N, int H, int W, int kernel_h, int kernel_w,
                   int stride_h, int stride_w, int pad_h, int pad_w,
                   int dilation_h, int dilation_w, int group, int group_channels,
                   float offset_scale, int remove_center, int om_channels,
                   int dtype, void *stream);

/*
 * DCNv3-compatible variants (walkthrough section 1.2 recap equation with the
 * softmax that section 2.1 removes): with softmax = 1 each (pixel, group)'s
 * K masks are logits, and the operation uses
 *   p_gk = exp(m_gk) / sum_j exp(m_gj)      (over all K points)
 * in place of m_gk.  The backward's mask gradient is then taken with respect
 * to the logits: dL/dm_gk = p_gk * (dL/dp_gk - sum_j p_gj * dL/dp_gj).
 * softmax = 0 is exactly dcnv4_forward / dcnv4_backward.  The masks must be
 * finite.  Arguments, layouts, ownership and errors as for the plain calls;
 * additionally PARAM if softmax is not 0 or 1, and UNSUPPORTED for softmax =
 * 1 with a geometry the LDS-tiled kernels do not cover (group_channels *
 * sizeof(dtype) a power-of-two multiple of 16 bytes, K <= 25).
 */
DCNV4_API int dcnv4_forward_ex(const void *value, const void *offset_mask, void *output,
                     int N, int H, int W, int kernel_h, int kernel_w,
                     int stride_h, int stride_w, int pad_h, int pad_w,
                     int dilation_h, int dilation_w, int group, int group_channels,
                     float offset_scale, int remove_center, int om_channels,
                     int softmax, int dtype, void *stream);

DCNV4_API int dcnv4_backward_ex(const void *value, const void *offset_mask, const void *grad_output,
                      void *grad_value, void *grad_offset_mask,
                      int N, int H, int W, int kernel_h, int kernel_w,
                      int stride_h, int stride_w, int pad_h, int pad_w,
                      int dilation_h, int dilation_w, int group, int group_channels,
                      float offset_scale, int remove_center, int om_channels,
                      int softmax, int dtype, void *stream);

#ifdef __cplusplus
}
#endif

#endif /* DCNV4_H */
