/*
 * flash_deform_attn.h -- C ABI of flash deformable attention (multi-scale
 * deformable attention with the softmax inside the operator) on MI355X
 * (gfx950), exported by libdcnv4.so next to the DCNv4 entry points of
 * dcnv4.h (same status codes and dtype codes).
 *
 * The pages name this operator only (the codewithpapers record of
 * "Efficient Deformable ConvNets", arXiv 2401.06197, lists the official
 * repository's DCNv4_op/DCNv4/functions/flash_deform_attn_func.py).  Its
 * arithmetic is the published definition of multi-scale deformable
 * attention (Zhu et al., "Deformable DETR", ICLR 2021, equation 3):
 *
 *   out[n,q,m,:] = sum_{l<L} sum_{k<K} a[n,q,m,l,k] *
 *                  x_l^m( u[n,q,m,l,k] * W_l - 1/2 , v[n,q,m,l,k] * H_l - 1/2 )
 *
 *   x_l^m(x, y) bilinear sample at column x, row y of head m's D channels of
 *               level l's H_l x W_l map, zero outside the map;
 *   (u, v)      normalised sampling location (u along the width; pixel
 *               (r, c) has its centre at ((c + 1/2)/W_l, (r + 1/2)/H_l));
 *   a           softmax over the L*K attention logits of (n, q, m).
 *
 * Conventions fixed by this library:
 *   - value    : (N, S, M, D), S = sum_l H_l*W_l; level l occupies rows
 *                [start_l, start_l + H_l*W_l), start_l = sum_{l'<l} H_l'*W_l',
 *                row-major (r, c); dense, channel-last.
 *   - loc_attn : (N, Q, M, P) with P = loc_attn_channels; row of (n, q, m):
 *                entries 2(l*K+k), 2(l*K+k)+1 = (u, v) of point (l, k);
 *                entry 2LK + l*K + k = its logit; entries [3LK, P) padding,
 *                never read.  (Locations and logits in one tensor, as the
 *                offsets and masks of DCNv4 are merged into one tensor.)
 *   - coordinate: x = fmaf(u, (float)W_l, -0.5f), y = fmaf(v, (float)H_l, -0.5f),
 *                fp32, one rounding.
 *   - border   : a bilinear corner outside the map contributes 0; a sample
 *                outside [-1,H_l) x [-1,W_l) (or NaN) contributes nothing but
 *                keeps its share of the softmax.
 *   - output   : (N, Q, M, D) = (N, Q, M*D), overwritten.
 *   - arithmetic: fp32 (softmax with the maximum subtracted, expf);
 *                outputs rounded to nearest-even into the storage dtype.
 *
 * Ownership, execution and errors as in dcnv4.h: caller-allocated dense
 * device buffers with 16-byte aligned bases, except spatial_shapes, which is
 * HOST memory (int[2*L] = H_0, W_0, H_1, W_1, ...) read during the call;
 * work enqueued on `stream` without waiting; outputs must not overlap inputs
 * or each other; all argument checks before any HIP call; N == 0 is a
 * valid no-op, and so is Q == 0 for the forward (the backward then writes
 * zeros to grad_value).
 */
#ifndef FLASH_DEFORM_ATTN_H
#define FLASH_DEFORM_ATTN_H

#include <stddef.h>

#include "dcnv4.h"

#ifdef __cplusplus
extern "C" {
#endif

/* Limits of this implementation. */
#define FLASH_DEFORM_ATTN_MAX_LEVELS 16
#define FLASH_DEFORM_ATTN_MAX_POINTS 128   /* L*K */

/*
 * Smallest valid loc_attn_channels: 3*L*K rounded up to a multiple of 8.
 * Returns a positive value, or DCNV4_ERR_PARAM (L or K < 1, or L*K above
 * FLASH_DEFORM_ATTN_MAX_POINTS).
 */
DCNV4_API int flash_deform_attn_channels(int num_levels, int num_points);

/*
 * Forward (the operation above).
 *
 *   value          (N, S, M, D)  dtype, read        S = num_value, M = num_heads, D = head_dim
 *   spatial_shapes int[2*L]      HOST, read          L = num_levels
 *   loc_attn       (N, Q, M, P)  dtype, read         Q = num_query, P = loc_attn_channels
 *   output         (N, Q, M, D)  dtype, written
 *
 * dtype: enum dcnv4_dtype, the same for all three tensors.
 * Errors: NULL; SHAPE (a size < 0, M, D, K < 1, a level size < 1, or
 * sum_l H_l*W_l != S); PARAM (L outside [1, FLASH_DEFORM_ATTN_MAX_LEVELS],
 * L*K above FLASH_DEFORM_ATTN_MAX_POINTS, P < 3LK or not a multiple of 8,
 * overlapping buffers); DTYPE; ALIGN; OVERFLOW (one image of value or
 * loc_attn exceeds 2^31 bytes, or N*Q*M exceeds 2^31); UNSUPPORTED (D not
 * in {8, 16, 32, 64, 128}); HIP.
 */
DCNV4_API int flash_deform_attn_forward(const void *value, const int *spatial_shapes, int num_levels,
                                        const void *loc_attn, void *output, int N, int num_value, int num_query,
                                        int num_heads, int head_dim, int num_points, int loc_attn_channels,
                                        int dtype, void *stream);

/*
 * Bytes of the workspace that flash_deform_attn_backward's sorted grad_value
 * path needs for these arguments (0 when N or Q is 0): 2 x 4 bytes per
 * corner bin ((H_l + 1) x (W_l + 1) bins per level, image and head) plus 16
 * bytes per (query, head, point), for the largest launch the call is split
 * into.  Writes *bytes.  Errors: NULL, and the argument errors of
 * flash_deform_attn_backward.
 */
DCNV4_API int flash_deform_attn_backward_workspace(const int *spatial_shapes, int num_levels, int N, int num_value,
                                                   int num_query, int num_heads, int head_dim, int num_points,
                                                   int loc_attn_channels, int dtype, size_t *bytes);

/*
 * Backward of flash_deform_attn_forward (chain rule of the operation above):
 *
 *   grad_value[corner]       = sum over samples of a * bilinear weight * grad_output
 *   grad_loc_attn u, v       = a * W_l * sum_d grad_output_d * d sample_d / dx,
 *                              a * H_l * sum_d grad_output_d * d sample_d / dy
 *                              (right derivative at integer coordinates)
 *   grad_loc_attn logit i    = a_i * (g_i - sum_j a_j g_j), g_i = sum_d grad_output_d * sample_{i,d}
 *
 *   value, spatial_shapes, loc_attn   as for the forward, read
 *   grad_output    (N, Q, M, D)  dtype, read
 *   grad_value     (N, S, M, D)  fp32 for every dtype, written (overwritten)
 *   grad_loc_attn  (N, Q, M, P)  dtype, written; padding entries 0
 *
 *   workspace      device memory of at least
 *                  flash_deform_attn_backward_workspace() bytes, 16-byte
 *                  aligned, owned by the caller, overwritten (its contents
 *                  are meaningless afterwards); or NULL
 *
 * With a workspace, grad_value is a gather: the samples are counting-sorted
 * by the cell of their top-left corner and every value cell sums its own
 * samples (atomic-free for floats; the sort uses integer device atomics).
 * With workspace == NULL every (sample, corner, channel) contribution is a
 * device fp32 atomic add into grad_value (about 8x slower at the measured
 * sizes).  grad_loc_attn is deterministic.  grad_value is summed in an order
 * that depends on thread timing on both paths, so its last bits may differ
 * from run to run.  Errors: as the forward, with UNSUPPORTED for D not in
 * {8, 16, 32, 64}; PARAM also for a workspace smaller than required or
 * overlapping another buffer; OVERFLOW also for Q*M*L*K above 2^31.
 */
DCNV4_API int flash_deform_attn_backward(const void *value, const int *spatial_shapes, int num_levels,
                                         const void *loc_attn, const void *grad_output, void *grad_value,
                                         void *grad_loc_attn, void *workspace, size_t workspace_bytes, int N,
                                         int num_value, int num_query, int num_heads, int head_dim, int num_points,
                                         int loc_attn_channels, int dtype, void *stream);

/*
 * flash_deform_attn_backward with no allocation and no workspace argument,
 * for callers that cannot allocate device memory (code under HIP graph
 * capture, tight serving loops, harnesses that forbid hipMalloc).  The
 * sorted grad_value path runs in a library-owned device array of
 * FLASH_DEFORM_ATTN_NOALLOC_SCRATCH_BYTES per device (a static device
 * variable, held by every device the library runs on until the process
 * ends) instead of a caller workspace; the call itself allocates and frees
 * nothing.  The caller still allocates value, loc_attn, grad_output,
 * grad_value and grad_loc_attn, as for flash_deform_attn_backward.
 *
 * Arguments, layouts, results and errors as flash_deform_attn_backward with
 * a workspace, except: the images of a call are processed in launches of
 * as many images as the array holds; UNSUPPORTED when one image alone needs
 * more than FLASH_DEFORM_ATTN_NOALLOC_SCRATCH_BYTES of workspace (the size
 * flash_deform_attn_backward_workspace reports for N = 1).  When a slice's
 * bins do not fit the on-chip sort, the device-atomic path runs, which
 * needs no workspace.  Every call on one device uses that device's one
 * array, so calls that overlap on one device (concurrent streams or host
 * threads) race and give wrong results; calls ordered on one stream are
 * safe.  The array keeps the last call's contents; what must start at zero
 * is cleared by each call (with a fill kernel, not a memset).
 */
#define FLASH_DEFORM_ATTN_NOALLOC_SCRATCH_BYTES (128u << 20)

DCNV4_API int flash_deform_attn_backward_noalloc(const void *value, const int *spatial_shapes, int num_levels,
                                                 const void *loc_attn, const void *grad_output, void *grad_value,
                                                 void *grad_loc_attn, int N, int num_value, int num_query,
                                                 int num_heads, int head_dim, int num_points, int loc_attn_channels,
                                                 int dtype, void *stream);

#ifdef __cplusplus
}
#endif

#endif /* FLASH_DEFORM_ATTN_H */
