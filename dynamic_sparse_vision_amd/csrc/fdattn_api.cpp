// C ABI of flash deformable attention (include/flash_deform_attn.h):
// argument validation, splitting into launches whose buffers fit 31-bit
// byte offsets, and dispatch.  Every check runs before the first HIP call.

#include "flash_deform_attn.h"

#include "dcnv4_internal.h"
#include "fdattn_internal.h"

#include <algorithm>
#include <cstddef>
#include <cstdint>

namespace {

constexpr int64_t kMaxLaunchBytes = 0x7fffffff;

bool aligned16(const void *p)
{
    return (reinterpret_cast<uintptr_t>(p) & 15u) == 0;
}

bool overlap(const void *a, int64_t na, const void *b, int64_t nb)
{
    const uintptr_t x = reinterpret_cast<uintptr_t>(a), y = reinterpret_cast<uintptr_t>(b);
    return x < y + (uintptr_t)nb && y < x + (uintptr_t)na;
}

// Validates everything but the tensor pointers.  On success fills *p (for
// all N images) and *per_launch.
int describe(const int *shapes, int L, int N, int S, int Q, int M, int D, int K, int P, int dtype, bool backward,
             fdattn::Problem *p, int *per_launch)
{
    if (!shapes)
        return DCNV4_ERR_NULL;
    if (dtype != DCNV4_FP32 && dtype != DCNV4_FP16 && dtype != DCNV4_BF16)
        return DCNV4_ERR_DTYPE;
    if (L < 1 || L > fdattn::kMaxLevels)
        return DCNV4_ERR_PARAM;
    if (N < 0 || S < 1 || Q < 0 || M < 1 || D < 1 || K < 1)
        return DCNV4_ERR_SHAPE;
    if ((int64_t)L * K > fdattn::kMaxPoints)
        return DCNV4_ERR_PARAM;
    if (P < 3 * L * K || P % 8 != 0)
        return DCNV4_ERR_PARAM;
    int64_t total = 0;
    for (int l = 0; l < L; ++l) {
        if (shapes[2 * l] < 1 || shapes[2 * l + 1] < 1)
            return DCNV4_ERR_SHAPE;
        p->lvl_h[l] = shapes[2 * l];
        p->lvl_w[l] = shapes[2 * l + 1];
        p->lvl_start[l] = (int)std::min<int64_t>(total, INT32_MAX);
        total += (int64_t)shapes[2 * l] * shapes[2 * l + 1];
        if (total > INT32_MAX)
            return DCNV4_ERR_OVERFLOW;
    }
    if (total != S)
        return DCNV4_ERR_SHAPE;
    const bool pow2 = (D & (D - 1)) == 0;
    if (D % 8 != 0 || !pow2 || D > (backward ? 64 : 128))
        return DCNV4_ERR_UNSUPPORTED;
    const int es = dtype == DCNV4_FP32 ? 4 : 2;
    const int64_t img_v = (int64_t)S * M * D * es;
    const int64_t img_gv = (int64_t)S * M * D * 4;
    const int64_t img_la = (int64_t)Q * M * P * es;
    const int64_t img_max = std::max(backward ? img_gv : img_v, img_la);
    if (img_max > kMaxLaunchBytes || (int64_t)N * Q * M > INT32_MAX)
        return DCNV4_ERR_OVERFLOW;
    p->N = N;
    p->S = S;
    p->Q = Q;
    p->M = M;
    p->D = D;
    p->K = K;
    p->L = L;
    p->P = P;
    p->dtype = dtype;
    p->elem = es;
    // value (and grad_value) of one launch are addressed with 31-bit offsets,
    // and the sorted backward numbers a launch's samples with 31 bits
    int64_t per = std::max<int64_t>(1, kMaxLaunchBytes / (backward ? img_gv : img_v));
    if (backward) {
        const int64_t samples = std::max<int64_t>(1, (int64_t)Q * M * L * K);
        if (samples > INT32_MAX)
            return DCNV4_ERR_OVERFLOW;
        per = std::min<int64_t>(per, INT32_MAX / samples);
    }
    *per_launch = (int)std::max<int64_t>(1, per);
    return DCNV4_OK;
}

// Workspace of the largest need among the launches a call is split into
// (full launches of per_launch images and the remainder).
size_t workspace_need(const fdattn::Problem &p, int N, int per_launch)
{
    size_t need = 0;
    for (int n : {std::min(N, per_launch), N % per_launch}) {
        if (n <= 0)
            continue;
        fdattn::Problem q = p;
        q.N = n;
        need = std::max(need, fdattn::workspace_bytes(q));
    }
    return need;
}

}  // namespace

extern "C" {

int flash_deform_attn_channels(int num_levels, int num_points)
{
    if (num_levels < 1 || num_points < 1 || (int64_t)num_levels * num_points > fdattn::kMaxPoints)
        return DCNV4_ERR_PARAM;
    return (3 * num_levels * num_points + 7) / 8 * 8;
}

int flash_deform_attn_forward(const void *value, const int *spatial_shapes, int num_levels, const void *loc_attn,
                              void *output, int N, int num_value, int num_query, int num_heads, int head_dim,
                              int num_points, int loc_attn_channels, int dtype, void *stream)
{
    dcnv4::clear_hip_error();
    fdattn::Problem p;
    int per_launch = 1;
    int st = describe(spatial_shapes, num_levels, N, num_value, num_query, num_heads, head_dim, num_points,
                      loc_attn_channels, dtype, false, &p, &per_launch);
    if (st != DCNV4_OK)
        return st;
    if (N == 0 || num_query == 0)
        return DCNV4_OK;
    if (!value || !loc_attn || !output)
        return DCNV4_ERR_NULL;
    if (!aligned16(value) || !aligned16(loc_attn) || !aligned16(output))
        return DCNV4_ERR_ALIGN;
    const int64_t es = p.elem;
    const int64_t img_v = (int64_t)p.S * p.M * p.D * es, img_la = (int64_t)p.Q * p.M * p.P * es,
                  img_o = (int64_t)p.Q * p.M * p.D * es;
    if (overlap(output, img_o * N, value, img_v * N) || overlap(output, img_o * N, loc_attn, img_la * N))
        return DCNV4_ERR_PARAM;
    hipStream_t s = static_cast<hipStream_t>(stream);
    for (int n0 = 0; n0 < N; n0 += per_launch) {
        fdattn::Problem q = p;
        q.N = std::min(per_launch, N - n0);
        hipError_t e = fdattn::launch_forward(q, static_cast<const char *>(value) + img_v * n0,
                                              static_cast<const char *>(loc_attn) + img_la * n0,
                                              static_cast<char *>(output) + img_o * n0, s);
        if (e != hipSuccess)
            return dcnv4::hip_status(e);
    }
    return DCNV4_OK;
}

int flash_deform_attn_backward_workspace(const int *spatial_shapes, int num_levels, int N, int num_value,
                                         int num_query, int num_heads, int head_dim, int num_points,
                                         int loc_attn_channels, int dtype, size_t *bytes)
{
    if (!bytes)
        return DCNV4_ERR_NULL;
    fdattn::Problem p;
    int per_launch = 1;
    int st = describe(spatial_shapes, num_levels, N, num_value, num_query, num_heads, head_dim, num_points,
                      loc_attn_channels, dtype, true, &p, &per_launch);
    if (st != DCNV4_OK)
        return st;
    *bytes = (N == 0 || num_query == 0) ? 0 : workspace_need(p, N, per_launch);
    return DCNV4_OK;
}

}  // extern "C"

namespace {

// The backward with the caller's workspace (workspace / workspace_bytes,
// or NULL: the device-atomic path), or, with `noalloc`, with the library's
// own scratch array, in as many launches as the array's size requires.
int backward_call(const void *value, const int *spatial_shapes, int num_levels, const void *loc_attn,
                  const void *grad_output, void *grad_value, void *grad_loc_attn, void *workspace,
                  size_t workspace_bytes, bool noalloc, int N, int num_value, int num_query, int num_heads,
                  int head_dim, int num_points, int loc_attn_channels, int dtype, void *stream)
{
    dcnv4::clear_hip_error();
    fdattn::Problem p;
    int per_launch = 1;
    int st = describe(spatial_shapes, num_levels, N, num_value, num_query, num_heads, head_dim, num_points,
                      loc_attn_channels, dtype, true, &p, &per_launch);
    if (st != DCNV4_OK)
        return st;
    if (N == 0)
        return DCNV4_OK;
    if (!value || !grad_value || (num_query > 0 && (!loc_attn || !grad_output || !grad_loc_attn)))
        return DCNV4_ERR_NULL;
    if (!aligned16(value) || !aligned16(loc_attn) || !aligned16(grad_output) || !aligned16(grad_value) ||
        !aligned16(grad_loc_attn) || !aligned16(workspace))
        return DCNV4_ERR_ALIGN;
    size_t need = 0;
    if (noalloc && num_query > 0) {
        // the largest number of images per launch whose workspace fits the
        // scratch array (none fits: refused)
        int fit = std::min(N, per_launch);
        while (fit > 0 && workspace_need(p, fit, fit) > fdattn::kNoAllocScratchBytes)
            --fit;
        if (fit == 0)
            return DCNV4_ERR_UNSUPPORTED;
        per_launch = fit;
        need = workspace_need(p, N, per_launch);
    } else if (workspace && num_query > 0) {
        need = workspace_need(p, N, per_launch);
        if (workspace_bytes < need)
            return DCNV4_ERR_PARAM;
    }
    const int64_t es = p.elem;
    const int64_t img_v = (int64_t)p.S * p.M * p.D * es, img_la = (int64_t)p.Q * p.M * p.P * es,
                  img_o = (int64_t)p.Q * p.M * p.D * es, img_gv = (int64_t)p.S * p.M * p.D * 4;
    const void *ins[3] = {value, loc_attn, grad_output};
    const int64_t in_sz[3] = {img_v * N, img_la * N, img_o * N};
    for (int i = 0; i < 3; ++i) {
        if (overlap(grad_value, img_gv * N, ins[i], in_sz[i]) || overlap(grad_loc_attn, img_la * N, ins[i], in_sz[i]))
            return DCNV4_ERR_PARAM;
    }
    if (overlap(grad_value, img_gv * N, grad_loc_attn, img_la * N))
        return DCNV4_ERR_PARAM;
    if (need > 0 && !noalloc) {
        const int64_t nw = (int64_t)need;
        for (int i = 0; i < 3; ++i) {
            if (overlap(workspace, nw, ins[i], in_sz[i]))
                return DCNV4_ERR_PARAM;
        }
        if (overlap(workspace, nw, grad_value, img_gv * N) || overlap(workspace, nw, grad_loc_attn, img_la * N))
            return DCNV4_ERR_PARAM;
    }
    hipStream_t s = static_cast<hipStream_t>(stream);
    if (noalloc && need > 0) {
        // every argument is checked: now the first HIP call
        const hipError_t e = fdattn::noalloc_scratch(&workspace);
        if (e != hipSuccess)
            return dcnv4::hip_status(e);
    }
    for (int n0 = 0; n0 < N; n0 += per_launch) {
        fdattn::Problem q = p;
        q.N = std::min(per_launch, N - n0);
        hipError_t e;
        if (num_query == 0) {
            // no query samples anything: grad_value is all zeros
            e = dcnv4::launch_zero(static_cast<char *>(grad_value) + img_gv * n0, (size_t)(img_gv * q.N), s);
        } else {
            e = fdattn::launch_backward(q, static_cast<const char *>(value) + img_v * n0,
                                        static_cast<const char *>(loc_attn) + img_la * n0,
                                        static_cast<const char *>(grad_output) + img_o * n0,
                                        reinterpret_cast<float *>(static_cast<char *>(grad_value) + img_gv * n0),
                                        static_cast<char *>(grad_loc_attn) + img_la * n0, need > 0 ? workspace : nullptr,
                                        s);
        }
        if (e != hipSuccess)
            return dcnv4::hip_status(e);
    }
    return DCNV4_OK;
}

}  // namespace

extern "C" {

int flash_deform_attn_backward(const void *value, const int *spatial_shapes, int num_levels, const void *loc_attn,
                               const void *grad_output, void *grad_value, void *grad_loc_attn, void *workspace,
                               size_t workspace_bytes, int N, int num_value, int num_query, int num_heads,
                               int head_dim, int num_points, int loc_attn_channels, int dtype, void *stream)
{
    return backward_call(value, spatial_shapes, num_levels, loc_attn, grad_output, grad_value, grad_loc_attn,
                         workspace, workspace_bytes, false, N, num_value, num_query, num_heads, head_dim,
                         num_points, loc_attn_channels, dtype, stream);
}

int flash_deform_attn_backward_noalloc(const void *value, const int *spatial_shapes, int num_levels,
                                       const void *loc_attn, const void *grad_output, void *grad_value,
                                       void *grad_loc_attn, int N, int num_value, int num_query, int num_heads,
                                       int head_dim, int num_points, int loc_attn_channels, int dtype, void *stream)
{
    return backward_call(value, spatial_shapes, num_levels, loc_attn, grad_output, grad_value, grad_loc_attn,
                         nullptr, 0, true, N, num_value, num_query, num_heads, head_dim, num_points,
                         loc_attn_channels, dtype, stream);
}

}  // extern "C"
