// C ABI of libdcnv4.so: argument validation, launch planning and dispatch.
// Every check runs before the first HIP call, so a rejected call has no side
// effects.  The operation itself is specified in include/dcnv4.h.

#include "dcnv4.h"
#include "dcnv4_internal.h"

#include <algorithm>
#include <cmath>
#include <cstdint>
#include <cstdio>
#include <cstring>

namespace dcnv4 {
namespace {

thread_local char g_last_hip_error[256] = "";

constexpr int64_t kMaxBytesPerLaunch = 0x7fffffff;   // 31-bit byte offsets
constexpr int kMaxThreads = 256;
constexpr int kMaxLds = 64 * 1024;
constexpr int kTargetLds = 48 * 1024;

int elem_size(int dtype)
{
    return dtype == DCNV4_FP32 ? 4 : 2;
}

bool ranges_overlap(const void *a, int64_t na, const void *b, int64_t nb)
{
    const uintptr_t x = reinterpret_cast<uintptr_t>(a), y = reinterpret_cast<uintptr_t>(b);
    return x < y + (uintptr_t)nb && y < x + (uintptr_t)na;
}

int output_size_1d(int in, int k, int s, int p, int d, int *out)
{
    const int64_t span = (int64_t)d * (k - 1) + 1;
    const int64_t num = (int64_t)in + 2 * (int64_t)p - span;
    if (num < 0) {
        *out = 0;
        return DCNV4_ERR_SHAPE;
    }
    const int64_t o = num / s + 1;
    if (o > INT32_MAX)
        return DCNV4_ERR_OVERFLOW;
    *out = (int)o;
    return DCNV4_OK;
}

// Validate scalar arguments and fill a Problem.  No pointer is looked at.
int describe(int N, int H, int W, int kh, int kw, int sh, int sw, int ph, int pw, int dh, int dw,
             int group, int group_channels, float offset_scale, int remove_center, int om_channels,
             int dtype, Problem *p)
{
    if (dtype != DCNV4_FP32 && dtype != DCNV4_FP16 && dtype != DCNV4_BF16)
        return DCNV4_ERR_DTYPE;
    if (N < 0 || H < 1 || W < 1)
        return DCNV4_ERR_SHAPE;
    if (kh < 1 || kw < 1 || sh < 1 || sw < 1 || dh < 1 || dw < 1 || ph < 0 || pw < 0)
        return DCNV4_ERR_PARAM;
    if (group < 1 || group_channels < 1)
        return DCNV4_ERR_PARAM;
    if (remove_center != 0 && remove_center != 1)
        return DCNV4_ERR_PARAM;
    if (remove_center && (kh % 2 == 0 || kw % 2 == 0 || kh * (int64_t)kw == 1))
        return DCNV4_ERR_PARAM;
    if (!std::isfinite(offset_scale))
        return DCNV4_ERR_PARAM;
    if ((int64_t)kh * kw > 4096)
        return DCNV4_ERR_UNSUPPORTED;
    const int K = kh * kw - remove_center;
    const int64_t C = (int64_t)group * group_channels;
    if (C > INT32_MAX / 4)
        return DCNV4_ERR_OVERFLOW;
    int Ho = 0, Wo = 0;
    int st = output_size_1d(H, kh, sh, ph, dh, &Ho);
    if (st != DCNV4_OK)
        return st;
    st = output_size_1d(W, kw, sw, pw, dw, &Wo);
    if (st != DCNV4_OK)
        return st;
    if (Ho < 1 || Wo < 1)
        return DCNV4_ERR_SHAPE;
    const int64_t need = 3 * (int64_t)group * K;
    if (om_channels < need || om_channels % 8 != 0)
        return DCNV4_ERR_PARAM;
    const int es = elem_size(dtype);
    // one image of each tensor must be addressable with 31-bit byte offsets
    const int64_t img_value = (int64_t)H * W * C * es;
    const int64_t img_om = (int64_t)Ho * Wo * om_channels * es;
    const int64_t img_out = (int64_t)Ho * Wo * C * es;
    const int64_t img_grad_om = (int64_t)Ho * Wo * om_channels * 4;
    if (img_value > kMaxBytesPerLaunch || img_om > kMaxBytesPerLaunch || img_out > kMaxBytesPerLaunch ||
        img_grad_om > kMaxBytesPerLaunch)
        return DCNV4_ERR_OVERFLOW;
    if ((int64_t)N * Ho * Wo > INT32_MAX)
        return DCNV4_ERR_OVERFLOW;
    p->N = N;
    p->H = H;
    p->W = W;
    p->Ho = Ho;
    p->Wo = Wo;
    p->kh = kh;
    p->kw = kw;
    p->sh = sh;
    p->sw = sw;
    p->ph = ph;
    p->pw = pw;
    p->dh = dh;
    p->dw = dw;
    p->G = group;
    p->Cg = group_channels;
    p->C = (int)C;
    p->K = K;
    p->P = om_channels;
    p->remove_center = remove_center;
    p->dtype = dtype;
    p->elem = es;
    p->offset_scale = offset_scale;
    return DCNV4_OK;
}

int64_t image_bytes_max(const Problem &p, bool backward)
{
    int64_t b = (int64_t)p.H * p.W * p.C * (backward ? 4 : p.elem);
    const int64_t om = (int64_t)p.Ho * p.Wo * p.P * (backward ? 4 : p.elem);
    const int64_t out = (int64_t)p.Ho * p.Wo * p.C * (backward ? 4 : p.elem);
    if (om > b)
        b = om;
    if (out > b)
        b = out;
    return b;
}

// Blocks of whole pixels with all their groups; shrink the pixel count until
// the staged offset_mask rows fit the LDS budget.
int plan_common(const Problem &p, int dp, int lds_rows_per_pixel_bytes, Plan *plan)
{
    plan->dp = dp;
    plan->lanes = p.Cg / dp;
    const int gl = p.G * plan->lanes;
    if (gl > kMaxThreads)
        return DCNV4_ERR_UNSUPPORTED;
    int ppb = kMaxThreads / gl;
    while (ppb > 1 && ppb * lds_rows_per_pixel_bytes > kTargetLds)
        ppb = (ppb + 1) / 2;
    if (ppb * (int64_t)lds_rows_per_pixel_bytes > kMaxLds)
        return DCNV4_ERR_UNSUPPORTED;
    plan->pix_per_block = ppb;
    plan->threads = ppb * gl;
    plan->lds_bytes = ppb * lds_rows_per_pixel_bytes;
    return DCNV4_OK;
}

}  // namespace

int plan_forward(const Problem &p, Plan *plan)
{
    if ((p.Cg * p.elem) % 16 != 0)
        return DCNV4_ERR_UNSUPPORTED;
    // channels per thread: up to 16, and whole 128-bit vectors
    int dp = 0;
    for (int cand : {16, 8, 4}) {
        if (p.Cg % cand == 0 && (cand * p.elem) % 16 == 0) {
            dp = cand;
            break;
        }
    }
    if (dp == 0)
        return DCNV4_ERR_UNSUPPORTED;
    int st = plan_common(p, dp, p.P * p.elem, plan);
    if (st != DCNV4_OK)
        return st;
    plan->images_per_launch = (int)(kMaxBytesPerLaunch / image_bytes_max(p, false));
    return DCNV4_OK;
}

int plan_backward(const Problem &p, Plan *plan)
{
    if (p.dtype != DCNV4_FP32)
        return DCNV4_ERR_UNSUPPORTED;
    if ((p.Cg * 4) % 16 != 0)
        return DCNV4_ERR_UNSUPPORTED;
    // lanes per (pixel, group) must be a power of two for the butterfly
    // reduction; prefer 4-channel lanes (denser atomics per cache line).
    int dp = 0;
    for (int cand : {4, 8, 16}) {
        const int lanes = p.Cg / cand;
        if (p.Cg % cand == 0 && lanes <= 64 && (lanes & (lanes - 1)) == 0) {
            dp = cand;
            break;
        }
    }
    if (dp == 0)
        return DCNV4_ERR_UNSUPPORTED;
    int st = plan_common(p, dp, 2 * p.P * 4, plan);
    if (st != DCNV4_OK)
        return st;
    plan->images_per_launch = (int)(kMaxBytesPerLaunch / image_bytes_max(p, true));
    return DCNV4_OK;
}

namespace {

bool pow2(int v)
{
    return v > 0 && (v & (v - 1)) == 0;
}

int ilog2(int v)
{
    int s = 0;
    while ((1 << s) < v)
        ++s;
    return s;
}

// Output tile for halo radius R: th x tw pixels with `lanes` threads per
// pixel, at most 256 threads and at least two waves (unless the map is
// smaller).  Cost, in 16-byte LDS operations: corner gathers of every wave
// slot (partial waves count in full) plus three per staged region vector.
void choose_out_tile(const Problem &p, int lanes, int nvl, int nvp, int R, int *th, int *tw)
{
    const long min_threads = std::min<long>(128, (long)p.Ho * p.Wo * lanes);
    double best = -1;
    for (int w = 1; w <= 64 && w <= p.Wo; ++w) {
        for (int h = 1; h <= 64 && h <= p.Ho; ++h) {
            const int threads = h * w * lanes;
            if (threads > 256)
                break;
            if (threads < min_threads)
                continue;
            const double blocks = (double)((p.Ho + h - 1) / h) * ((p.Wo + w - 1) / w);
            const double rh = (h - 1) * p.sh + (p.kh - 1) * p.dh + 2 * R + 2;
            const double rw = (w - 1) * p.sw + (p.kw - 1) * p.dw + 2 * R + 2;
            const double cost = blocks * ((threads + 63) / 64) * 64.0 * p.K * 4 * nvl + blocks * rh * rw * nvp * 3;
            if (best < 0 || cost < best) {
                best = cost;
                *th = h;
                *tw = w;
            }
        }
    }
}

// Cell tile of the grad_value kernel (one thread per cell, at most 256):
// minimise the samples evaluated, i.e. blocks x source pixels x K, plus a
// fixed per-block cost.
void choose_cell_tile(const Problem &p, int R, int *ch, int *cw)
{
    double best = -1;
    for (int w = 1; w <= 256 && w <= p.W; ++w) {
        for (int h = 1; h <= 256 && h <= p.H; ++h) {
            if (h * w > 256)
                break;
            const double blocks = (double)((p.H + h - 1) / h) * ((p.W + w - 1) / w);
            const double sh = (double)(h + (p.kh - 1) * p.dh + 2 * R + 2) / p.sh + 1;
            const double sw = (double)(w + (p.kw - 1) * p.dw + 2 * R + 2) / p.sw + 1;
            const double cost = blocks * (sh * sw * p.K + 2048);
            if (best < 0 || cost < best) {
                best = cost;
                *ch = h;
                *cw = w;
            }
        }
    }
}

// Fill the LDS region geometry for halo radius R; returns total LDS bytes.
int tile_lds(const Problem &p, TilePlan *tp, int R, int elem)
{
    tp->R = R;
    tp->rh = (tp->th - 1) * p.sh + (p.kh - 1) * p.dh + 2 * R + 2;
    tp->rw = (tp->tw - 1) * p.sw + (p.kw - 1) * p.dw + 2 * R + 2;
    // a group's 3K entries, widened to whole dwords (2-byte entries may start
    // mid-dword)
    tp->om_dw = elem == 4 ? 3 * p.K : (3 * p.K + 2) / 2;
    const int om = tp->th * tp->tw * tp->om_dw * 4;
    tp->om_lds_bytes = (om + 15) / 16 * 16;
    tp->lds_bytes = tp->om_lds_bytes + tp->rh * tp->rw * tp->nvp * 16;
    return tp->lds_bytes;
}

constexpr int kTiledMaxLds = 80 * 1024;

int plan_tiled_common(const Problem &p, int elem, int r_max, int lds_budget, TilePlan *tp)
{
    if ((p.Cg * elem) % 16 != 0)
        return DCNV4_ERR_UNSUPPORTED;
    tp->nvp = p.Cg * elem / 16;
    if (!pow2(tp->nvp))
        return DCNV4_ERR_UNSUPPORTED;
    int dp = 0;
    for (int cand : {16, 8, 4}) {
        if (p.Cg % cand == 0 && (cand * elem) % 16 == 0) {
            dp = cand;
            break;
        }
    }
    if (dp == 0)
        return DCNV4_ERR_UNSUPPORTED;
    tp->dp = dp;
    tp->lanes = p.Cg / dp;
    if (!pow2(tp->lanes) || tp->lanes > 64)
        return DCNV4_ERR_UNSUPPORTED;
    // 16 LDS banks of 16 bytes: rotate the vector index by higher pixel bits
    tp->swz_mask = (tp->nvp >= 2) ? (tp->nvp < 16 ? tp->nvp : 16) - 1 : 0;
    tp->swz_shift = tp->nvp < 16 ? ilog2(16 / tp->nvp) : 0;
    const int nvl = dp * elem / 16;
    // the largest halo radius whose best tile fits the LDS budget
    for (int R = r_max; R >= 1; --R) {
        choose_out_tile(p, tp->lanes, nvl, tp->nvp, R, &tp->th, &tp->tw);
        if (tile_lds(p, tp, R, elem) <= lds_budget) {
            // whole waves: the kernels' staging loops stride by 64 lanes
            tp->threads = (tp->th * tp->tw * tp->lanes + 63) / 64 * 64;
            tp->tiles_y = (p.Ho + tp->th - 1) / tp->th;
            tp->tiles_x = (p.Wo + tp->tw - 1) / tp->tw;
            tp->images_per_launch = 0;
            return DCNV4_OK;
        }
    }
    return DCNV4_ERR_UNSUPPORTED;
}

}  // namespace

int plan_forward_tiled(const Problem &p, TilePlan *tp)
{
    *tp = TilePlan{};
    // fp32 rows are twice as wide: a smaller halo keeps two blocks per CU
    const int r_max = p.elem == 4 ? 5 : 8;
    const int budget = p.elem == 4 ? kTiledMaxLds : 64 * 1024;
    int st = plan_tiled_common(p, p.elem, r_max, budget, tp);
    if (st != DCNV4_OK)
        return st;
    tp->images_per_launch = (int)(kMaxBytesPerLaunch / image_bytes_max(p, false));
    return DCNV4_OK;
}

int plan_backward_tiled(const Problem &p, TilePlan *tp)
{
    *tp = TilePlan{};
    if (p.dtype != DCNV4_FP32)
        return DCNV4_ERR_UNSUPPORTED;
    if (p.Cg != 4 && p.Cg != 8 && p.Cg != 16 && p.Cg != 32)
        return DCNV4_ERR_UNSUPPORTED;
    int st = plan_tiled_common(p, 4, 5, kTiledMaxLds, tp);
    if (st != DCNV4_OK)
        return st;
    // cell tiles for grad_value: one thread per cell, at most 256 cells
    choose_cell_tile(p, tp->R, &tp->ch, &tp->cw);
    tp->ctiles_y = (p.H + tp->ch - 1) / tp->ch;
    tp->ctiles_x = (p.W + tp->cw - 1) / tp->cw;
    // a batch holds at most 1024 samples (4 per thread), i.e. 4096 corner
    // records, and at most 128 source pixels (their grad_out rows sit in LDS)
    tp->src_batch = std::min(1024 / p.K, 128);
    if (tp->src_batch < 1)
        return DCNV4_ERR_UNSUPPORTED;
    tp->max_records = 4096;
    tp->splat_lds_bytes = 3 * 256 * 4 + 16 + tp->max_records * 8 + tp->src_batch * p.Cg * 4;
    tp->images_per_launch = (int)(kMaxBytesPerLaunch / image_bytes_max(p, true));
    return DCNV4_OK;
}

}  // namespace dcnv4

using namespace dcnv4;

namespace {

int hip_status(hipError_t e)
{
    if (e == hipSuccess)
        return DCNV4_OK;
    std::snprintf(g_last_hip_error, sizeof g_last_hip_error, "%s: %s", hipGetErrorName(e),
                  hipGetErrorString(e));
    return DCNV4_ERR_HIP;
}

bool aligned16(const void *p)
{
    return (reinterpret_cast<uintptr_t>(p) & 15u) == 0;
}

}  // namespace

extern "C" {

int dcnv4_abi_version(void)
{
    return DCNV4_ABI_VERSION;
}

const char *dcnv4_status_string(int status)
{
    switch (status) {
    case DCNV4_OK: return "ok";
    case DCNV4_ERR_NULL: return "a required pointer is NULL";
    case DCNV4_ERR_SHAPE: return "invalid or empty shape";
    case DCNV4_ERR_PARAM: return "invalid parameter";
    case DCNV4_ERR_DTYPE: return "unknown dtype";
    case DCNV4_ERR_ALIGN: return "pointer not 16-byte aligned";
    case DCNV4_ERR_UNSUPPORTED: return "unsupported configuration";
    case DCNV4_ERR_OVERFLOW: return "size exceeds the index range";
    case DCNV4_ERR_HIP: return "HIP runtime error";
    default: return "unknown status";
    }
}

const char *dcnv4_last_hip_error(void)
{
    return g_last_hip_error;
}

int dcnv4_output_size(int H, int W, int kernel_h, int kernel_w, int stride_h, int stride_w, int pad_h,
                      int pad_w, int dilation_h, int dilation_w, int *Ho, int *Wo)
{
    if (!Ho || !Wo)
        return DCNV4_ERR_NULL;
    if (kernel_h < 1 || kernel_w < 1 || stride_h < 1 || stride_w < 1 || dilation_h < 1 || dilation_w < 1 ||
        pad_h < 0 || pad_w < 0)
        return DCNV4_ERR_PARAM;
    if (H < 1 || W < 1)
        return DCNV4_ERR_SHAPE;
    int st = output_size_1d(H, kernel_h, stride_h, pad_h, dilation_h, Ho);
    if (st != DCNV4_OK)
        return st;
    st = output_size_1d(W, kernel_w, stride_w, pad_w, dilation_w, Wo);
    if (st != DCNV4_OK)
        return st;
    return (*Ho < 1 || *Wo < 1) ? DCNV4_ERR_SHAPE : DCNV4_OK;
}

int dcnv4_om_channels(int group, int kernel_h, int kernel_w, int remove_center)
{
    if (group < 1 || kernel_h < 1 || kernel_w < 1 || (remove_center != 0 && remove_center != 1))
        return DCNV4_ERR_PARAM;
    if (remove_center && (kernel_h % 2 == 0 || kernel_w % 2 == 0 || kernel_h * (int64_t)kernel_w == 1))
        return DCNV4_ERR_PARAM;
    const int64_t K = (int64_t)kernel_h * kernel_w - remove_center;
    const int64_t P = (3 * group * K + 7) / 8 * 8;
    if (P > INT32_MAX)
        return DCNV4_ERR_PARAM;
    return (int)P;
}

int dcnv4_forward(const void *value, const void *offset_mask, void *output, int N, int H, int W, int kernel_h,
                  int kernel_w, int stride_h, int stride_w, int pad_h, int pad_w, int dilation_h, int dilation_w,
                  int group, int group_channels, float offset_scale, int remove_center, int om_channels, int dtype,
                  void *stream)
{
    g_last_hip_error[0] = '\0';
    Problem p;
    int st = describe(N, H, W, kernel_h, kernel_w, stride_h, stride_w, pad_h, pad_w, dilation_h, dilation_w, group,
                      group_channels, offset_scale, remove_center, om_channels, dtype, &p);
    if (st != DCNV4_OK)
        return st;
    Plan plan;
    TilePlan tp;
    const bool tiled = plan_forward_tiled(p, &tp) == DCNV4_OK;
    st = plan_forward(p, &plan);
    if (st != DCNV4_OK && !tiled)
        return st;
    if (N == 0)
        return DCNV4_OK;
    if (!value || !offset_mask || !output)
        return DCNV4_ERR_NULL;
    if (!aligned16(value) || !aligned16(offset_mask) || !aligned16(output))
        return DCNV4_ERR_ALIGN;
    const int64_t es = p.elem;
    const int64_t img_v = (int64_t)p.H * p.W * p.C * es, img_om = (int64_t)p.Ho * p.Wo * p.P * es,
                  img_o = (int64_t)p.Ho * p.Wo * p.C * es;
    const int64_t nv = img_v * N, nom = img_om * N, no = img_o * N;
    if (ranges_overlap(output, no, value, nv) || ranges_overlap(output, no, offset_mask, nom))
        return DCNV4_ERR_PARAM;
    hipStream_t s = static_cast<hipStream_t>(stream);
    const int per_launch = tiled ? tp.images_per_launch : plan.images_per_launch;
    for (int n0 = 0; n0 < N; n0 += per_launch) {
        Problem q = p;
        q.N = std::min(per_launch, N - n0);
        const void *v = static_cast<const char *>(value) + img_v * n0;
        const void *om = static_cast<const char *>(offset_mask) + img_om * n0;
        void *o = static_cast<char *>(output) + img_o * n0;
        hipError_t e = tiled ? launch_forward_tiled(q, tp, v, om, o, s) : launch_forward_general(q, plan, v, om, o, s);
        if (e != hipSuccess)
            return hip_status(e);
    }
    return DCNV4_OK;
}

int dcnv4_backward(const void *value, const void *offset_mask, const void *grad_output, void *grad_value,
                   void *grad_offset_mask, int N, int H, int W, int kernel_h, int kernel_w, int stride_h,
                   int stride_w, int pad_h, int pad_w, int dilation_h, int dilation_w, int group,
                   int group_channels, float offset_scale, int remove_center, int om_channels, int dtype,
                   void *stream)
{
    g_last_hip_error[0] = '\0';
    Problem p;
    int st = describe(N, H, W, kernel_h, kernel_w, stride_h, stride_w, pad_h, pad_w, dilation_h, dilation_w, group,
                      group_channels, offset_scale, remove_center, om_channels, dtype, &p);
    if (st != DCNV4_OK)
        return st;
    Plan plan;
    TilePlan tp;
    const bool tiled = plan_backward_tiled(p, &tp) == DCNV4_OK;
    st = plan_backward(p, &plan);
    if (st != DCNV4_OK && !tiled)
        return st;
    if (N == 0)
        return DCNV4_OK;
    if (!value || !offset_mask || !grad_output || !grad_value || !grad_offset_mask)
        return DCNV4_ERR_NULL;
    if (!aligned16(value) || !aligned16(offset_mask) || !aligned16(grad_output) || !aligned16(grad_value) ||
        !aligned16(grad_offset_mask))
        return DCNV4_ERR_ALIGN;
    const int64_t img_v = (int64_t)p.H * p.W * p.C * 4, img_om = (int64_t)p.Ho * p.Wo * p.P * 4,
                  img_o = (int64_t)p.Ho * p.Wo * p.C * 4;
    const int64_t nv = img_v * N, nom = img_om * N, no = img_o * N;
    const void *ins[3] = {value, offset_mask, grad_output};
    const int64_t in_sz[3] = {nv, nom, no};
    for (int i = 0; i < 3; ++i) {
        if (ranges_overlap(grad_value, nv, ins[i], in_sz[i]) || ranges_overlap(grad_offset_mask, nom, ins[i], in_sz[i]))
            return DCNV4_ERR_PARAM;
    }
    if (ranges_overlap(grad_value, nv, grad_offset_mask, nom))
        return DCNV4_ERR_PARAM;
    hipStream_t s = static_cast<hipStream_t>(stream);
    const int per_launch = tiled ? tp.images_per_launch : plan.images_per_launch;
    for (int n0 = 0; n0 < N; n0 += per_launch) {
        Problem q = p;
        q.N = std::min(per_launch, N - n0);
        const void *v = static_cast<const char *>(value) + img_v * n0;
        const void *om = static_cast<const char *>(offset_mask) + img_om * n0;
        const void *go = static_cast<const char *>(grad_output) + img_o * n0;
        void *gv = static_cast<char *>(grad_value) + img_v * n0;
        void *gom = static_cast<char *>(grad_offset_mask) + img_om * n0;
        hipError_t e = tiled ? launch_backward_tiled(q, tp, v, om, go, gv, gom, s)
                             : launch_backward_general(q, plan, v, om, go, gv, gom, s);
        if (e != hipSuccess)
            return hip_status(e);
    }
    return DCNV4_OK;
}

}  // extern "C"
