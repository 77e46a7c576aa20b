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
#include <mutex>
#include <vector>

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

// a * b for non-negative a, b, or INT64_MAX when that overflows
int64_t mul_sat(int64_t a, int64_t b)
{
    int64_t r;
    return __builtin_mul_overflow(a, b, &r) ? INT64_MAX : r;
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
    // (products saturate: H * W * C alone can exceed 64 bits)
    const int64_t img_value = mul_sat(mul_sat(H, W), C * es);
    const int64_t img_om = mul_sat(mul_sat(Ho, Wo), (int64_t)om_channels * es);
    const int64_t img_out = mul_sat(mul_sat(Ho, Wo), C * es);
    const int64_t img_grad_om = mul_sat(mul_sat(Ho, Wo), (int64_t)om_channels * 4);
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
    p->softmax = 0;
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

constexpr int kRowSlots = 512;        // a staged LDS row spans at most 8 x 64 slots
constexpr int kMaxTiledK = 25;        // grid points of the tiled kernels
#ifndef DCNV4_FWD_RMAX
#define DCNV4_FWD_RMAX 5
#endif
constexpr int kForwardRmax = DCNV4_FWD_RMAX;   // largest halo of the forward tiles
#ifndef DCNV4_FWD_RMAX_LARGE
#define DCNV4_FWD_RMAX_LARGE 7
#endif
constexpr int kForwardRmaxLarge = DCNV4_FWD_RMAX_LARGE;   // ... on large maps
#ifndef DCNV4_BWD_RMAX
#define DCNV4_BWD_RMAX 7
#endif
constexpr int kBackwardRmax = DCNV4_BWD_RMAX;  // near radius of the backward's grad_value cell tiles
#ifndef DCNV4_BWD_RMAX_LARGE
#define DCNV4_BWD_RMAX_LARGE 11
#endif
constexpr int kBackwardRmaxLarge = DCNV4_BWD_RMAX_LARGE;   // ... on large maps
#ifndef DCNV4_BWD_REGION_RMAX
#define DCNV4_BWD_REGION_RMAX 4
#endif
constexpr int kBackwardRegionRmax = DCNV4_BWD_REGION_RMAX;   // largest halo of the grad_offset_mask tiles
#ifndef DCNV4_BWD_REGION_RMAX_LARGE
#define DCNV4_BWD_REGION_RMAX_LARGE 6
#endif
#ifndef DCNV4_BWD_SLICE_LARGE
#define DCNV4_BWD_SLICE_LARGE 64
#endif
constexpr int kBackwardRegionRmaxLarge = DCNV4_BWD_REGION_RMAX_LARGE;   // ... on large maps
constexpr int kBackwardSliceLarge = DCNV4_BWD_SLICE_LARGE;   // pixel slice bytes of its blocks there
#ifndef DCNV4_TILED_LDS_KB
#define DCNV4_TILED_LDS_KB 80
#endif
constexpr int kTiledMaxLds = DCNV4_TILED_LDS_KB * 1024;
constexpr int kLdsPerCu = 160 * 1024;
// A block's LDS is allocated in 1280-byte units: 7-wave forward blocks of
// 54000 bytes averaged 10.5 resident waves per CU (two blocks fit, not three),
// 8-wave blocks of 50112 bytes 16 (three fit).
constexpr int kLdsGranule = 1280;
constexpr int kTileThreads = 512;
#ifndef DCNV4_CELL_LDS_KB
#define DCNV4_CELL_LDS_KB 78
#endif
constexpr int kCellTileLds = DCNV4_CELL_LDS_KB * 1024;   // two cell-tile blocks per CU
constexpr int kCellBinBytes = kCellBinSlots * 4 + (kCellThreads / 64) * 4;   // counters, scan scratch

// Upper bound of the source window width of a cell tile cw cells wide.
int window_cols(const Problem &p, int cw, int R)
{
    return (cw + 2 * R + (p.kw - 1) * p.dw + 1) / p.sw + 2;
}

int floor_div_h(int a, int b)
{
    const int q = a / b;
    return (a % b != 0 && ((a < 0) != (b < 0))) ? q - 1 : q;
}

// Source range [s0, s1) of a cell range starting at c0, `len` cells long,
// along one axis (the kernel's window: output pixels whose near samples can
// put a top-left corner in [c0 - 1, c0 + len - 1]).
void source_range(int c0, int len, int R, int pad, int kern, int dil, int stride, int out, int *s0, int *s1)
{
    *s0 = std::max(0, -floor_div_h(-(c0 - 1 - R + pad - (kern - 1) * dil), stride));
    *s1 = std::min(out, floor_div_h(c0 + len - 1 + R + pad, stride) + 1);
}

// Cell tile of the grad_value kernel: ch x cw cells, ch even, one thread
// per vertical pair.  Modelled cost, summed over the tiles of an image:
// per batch, the sample evaluation of its source waves plus a fixed part
// (staging, the scan, four barriers); per block, the three-run gathers of
// its pair waves (about 10 instructions per record of a 9-point sample).
bool choose_cell_tile(const Problem &p, int R, int src_cap, int gps, int *ch, int *cw)
{
    double best = -1;
    const int hmax = std::min(128, (p.H + 1) / 2 * 2);
    for (int w = 1; w <= 128 && w <= p.W; ++w) {
        const int sw_max = window_cols(p, w, R);
        if (sw_max > src_cap || sw_max * gps > kRowSlots)
            break;
        for (int h = 2; h <= hmax; h += 2) {
            if ((h / 2) * w > kCellThreads || (h + 1) * (w + 1) >= kCellBinSlots)
                break;
            const int pair_waves = ((h / 2) * w + 63) / 64;
            // tiles along each axis, grouped by source window size
            std::vector<std::pair<int, int>> rows, cols;   // (window size, tiles)
            auto windows = [&](int len, int size, int pad, int kern, int dil, int stride, int out,
                               std::vector<std::pair<int, int>> &acc) {
                for (int c0 = 0; c0 < size; c0 += len) {
                    int s0, s1;
                    source_range(c0, len, R, pad, kern, dil, stride, out, &s0, &s1);
                    const int n = std::max(0, s1 - s0);
                    bool found = false;
                    for (auto &e : acc)
                        if (e.first == n) {
                            ++e.second;
                            found = true;
                        }
                    if (!found)
                        acc.emplace_back(n, 1);
                }
            };
            windows(h, p.H, p.ph, p.kh, p.dh, p.sh, p.Ho, rows);
            windows(w, p.W, p.pw, p.kw, p.dw, p.sw, p.Wo, cols);
            double cost = 0;
            for (const auto &ry : rows) {
                for (const auto &cx : cols) {
                    const int sh = ry.first, sw = cx.first;
                    double blk = 400.0 + pair_waves * 90.0 * 4 * p.K;
                    if (sw > 0) {
                        const int br = std::max(1, src_cap / sw);
                        for (int r = 0; r < sh; r += br) {
                            const int nsrc = std::min(br, sh - r) * sw;
                            blk += 800.0 + ((nsrc + 63) / 64) * (40.0 * p.K + 60.0);
                        }
                    }
                    cost += blk * ry.second * cx.second;
                }
            }
            if (best < 0 || cost < best) {
                best = cost;
                *ch = h;
                *cw = w;
            }
        }
    }
    return best >= 0;
}

// The forward's LDS region of a tile along one axis: the tile's grid span
// plus a halo of R, clamped to the image plus a one-pixel zero border
// (-1 .. size); the kernel computes the same bounds (fwd_region).
int fwd_region_len(int t0, int t, int stride, int pad, int kern, int dil, int R, int size)
{
    const int lo_u = t0 * stride - pad - R;
    const int span = (t - 1) * stride + (kern - 1) * dil + 2 * R + 2;
    return std::min(lo_u + span, size + 1) - std::max(lo_u, -1);
}

// Largest region length over the tiles of one axis, and the sum of the
// region lengths (the staged pixels along that axis).
// The allocation holds at least 2 x 2 pixels: samples that are not near
// read the region's first footprint (with zero weights), also in a block
// whose clamped region is empty (a tile that sees only padding).
void fwd_region_stats(int out, int t, int stride, int pad, int kern, int dil, int R, int size, int *maxlen, long *sum)
{
    *maxlen = 2;
    *sum = 0;
    for (int t0 = 0; t0 < out; t0 += t) {
        const int len = fwd_region_len(t0, t, stride, pad, kern, dil, R, size);
        *maxlen = std::max(*maxlen, len);
        *sum += std::max(len, 0);
    }
}

// Output tiles: th x tw pixels of gb groups, `lanes` threads of dp
// channels per pixel and group, at most kTileThreads threads; the LDS holds
// the widest clamped region at pst 16-byte slots per pixel, and at least
// pixel_bytes per tile pixel (the backward's gradient rows; 0 for the
// forward).  Modelled time, summed over the tiles of an image: a lane-sample
// costs ~30 instructions plus one FMA per channel and corner, a staged
// region slot ~8; blocks run concurrently until `max_waves` share a CU
// (fewer when the LDS limits them).
bool choose_tile(const Problem &p, int lanes, int dp, int gb, int pst, int R, int lds_budget, int max_waves,
                 int pixel_bytes, int *th, int *tw, int *rh, int *rw)
{
    double best = -1;
    for (int w = 1; w <= 64 && w <= p.Wo; ++w) {
        int rwm;
        long rws;
        fwd_region_stats(p.Wo, w, p.sw, p.pw, p.kw, p.dw, R, p.W, &rwm, &rws);
        if (rwm * pst > kRowSlots)
            break;
        for (int h = 1; h <= 64 && h <= p.Ho; ++h) {
            const int threads = h * w * gb * lanes;
            if (threads > kTileThreads)
                break;
            int rhm;
            long rhs;
            fwd_region_stats(p.Ho, h, p.sh, p.ph, p.kh, p.dh, R, p.H, &rhm, &rhs);
            const int lds = std::max(rhm * rwm * pst * 16, h * w * pixel_bytes);
            if (lds > lds_budget)
                continue;
            const int waves = (threads + 63) / 64;
            const int per_cu = std::min(kLdsPerCu / ((lds + kLdsGranule - 1) / kLdsGranule * kLdsGranule),
                                        max_waves / waves);
            if (per_cu < 1)
                continue;
            const double occ = std::min(1.0, per_cu * waves / (double)max_waves);
            const double blocks = (double)((p.Ho + h - 1) / h) * ((p.Wo + w - 1) / w) * (p.G / gb);
            const double work = blocks * waves * 64.0 * p.K * (30 + 4 * dp) + (double)rhs * rws * pst * 8 * (p.G / gb);
            const double cost = work / occ;
            if (best < 0 || cost < best) {
                best = cost;
                *th = h;
                *tw = w;
                *rh = rhm;
                *rw = rwm;
            }
        }
    }
    return best >= 0;
}

// Output tiles of the forward and of the backward's grad_offset_mask
// kernel: channels per lane, groups per block (pixel slices of at most
// slice_bytes), halo radius (the largest up to r_max with a tile in the LDS
// budget) and the tile.  group_row_bytes: LDS per pixel and group beyond the
// value region (the backward's gradient rows; 0 for the forward).
int plan_out_tiles(const Problem &p, int r_max, int max_waves, int group_row_bytes, int slice_bytes, TilePlan *tp)
{
    // near-sample addresses take floors below 2^22 in magnitude
    if ((p.Cg * p.elem) % 16 != 0 || p.K > kMaxTiledK || p.H > (1 << 21) || p.W > (1 << 21))
        return DCNV4_ERR_UNSUPPORTED;
    tp->nvp = p.Cg * p.elem / 16;
    if (!pow2(tp->nvp))
        return DCNV4_ERR_UNSUPPORTED;
    // channels per lane: 16-bit pixels of 16 channels take one lane (two
    // 128-bit vectors per corner); fp32 takes 8 channels per lane
    int dp = 0;
    const int cands16[] = {16, 8}, cands32[] = {8, 4};
    for (int cand : (p.elem == 2 ? cands16 : cands32)) {
        if (p.Cg % cand == 0 && (cand * p.elem) % 16 == 0) {
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
    // groups per block: the largest power of two dividing G whose slices of
    // a pixel make at most slice_bytes (128: one whole cache line, so that
    // staging, offset/mask loads and output stores cover whole lines)
    tp->gb = 1;
    while (p.G % (2 * tp->gb) == 0 && 2 * tp->gb * tp->nvp * 16 <= slice_bytes)
        tp->gb *= 2;
    const int nvb = tp->gb * tp->nvp;
    tp->ps = nvb | 1;   // odd LDS pixel stride: random pixel reads spread over the banks
    for (int R = r_max; R >= 1; --R) {
        if (!choose_tile(p, tp->lanes, dp, tp->gb, tp->ps, R, kTiledMaxLds, max_waves, tp->gb * group_row_bytes,
                         &tp->th, &tp->tw, &tp->rh, &tp->rw))
            continue;
        tp->R = R;
        tp->lds_bytes = std::max(tp->rh * tp->rw * tp->ps * 16, tp->th * tp->tw * tp->gb * group_row_bytes);
        // whole waves: the staging loop takes rows per wave
        tp->threads = (tp->th * tp->tw * tp->gb * tp->lanes + 63) / 64 * 64;
        tp->tiles_y = (p.Ho + tp->th - 1) / tp->th;
        tp->tiles_x = (p.Wo + tp->tw - 1) / tp->tw;
        return DCNV4_OK;
    }
    return DCNV4_ERR_UNSUPPORTED;
}

// Large maps: at least this many pixels on the shorter side.  Offsets in
// pixels grow with the map, so there the output tiles take a wider halo with
// narrower pixel slices (at 128 bytes a halo of 7 leaves tiles too small),
// and the cell tiles a larger near radius.
constexpr int kLargeMapSide = 192;

bool large_map(const Problem &p)
{
    return std::min(p.H, p.W) >= kLargeMapSide;
}

int compute_forward_tiled(const Problem &p, TilePlan *tp)
{
    *tp = TilePlan{};
    const bool large = large_map(p);
    const int st = plan_out_tiles(p, large ? kForwardRmaxLarge : kForwardRmax, 24, 0, large ? 64 : 128, tp);
    if (st != DCNV4_OK)
        return st;
    tp->images_per_launch = (int)(kMaxBytesPerLaunch / image_bytes_max(p, false));
    return DCNV4_OK;
}

int compute_backward_tiled(const Problem &p, TilePlan *tp)
{
    *tp = TilePlan{};
    // grad_value cell tiles are instantiated for these channel counts
    const bool cg_ok = p.Cg == 8 || p.Cg == 16 || p.Cg == 32 || (p.Cg == 4 && p.elem == 4);
    if (!cg_ok)
        return DCNV4_ERR_UNSUPPORTED;
    // grad_offset_mask tiles: as the forward's, with the tile's gradient rows
    // (3K fp32 per pixel and group) in the same LDS at the end; the kernel
    // keeps more registers, so fewer waves share a CU
    const bool large = large_map(p);
    int st = plan_out_tiles(p, large ? kBackwardRegionRmaxLarge : kBackwardRegionRmax, 16, 3 * p.K * 4,
                            large ? kBackwardSliceLarge : 128, tp);
    if (st != DCNV4_OK)
        return st;
    // cell tiles for grad_value: LDS holds the bins, up to src_cap*K sorted
    // samples of 16 bytes and src_cap staged grad_output pixels
    tp->gps = (p.Cg * p.elem / 16) | 1;
    tp->rec_offset = kCellBinBytes;
    tp->src_cap = std::min(kCellThreads, (kCellTileLds - kCellBinBytes) / (16 * (p.K + tp->gps)));
    if (tp->src_cap < 1)
        return DCNV4_ERR_UNSUPPORTED;
    // The near radius of the cell tiles.  A sample beyond it costs the
    // grad_offset_mask kernel a device atomic per channel and corner; one
    // within it costs every cell tile whose source window holds its pixel,
    // and the windows grow with the radius.  Offsets in pixels grow with the
    // map, so the radius does too: 7 up to 95 pixels on the shorter side,
    // then one more per 32 pixels, up to 11 from 192 pixels.
    const int side = std::min(p.H, p.W);
    tp->Rc = std::min(kBackwardRmaxLarge, kBackwardRmax + std::max(0, (side - 64) / 32));
    while (!choose_cell_tile(p, tp->Rc, tp->src_cap, tp->gps, &tp->ch, &tp->cw))
        if (--tp->Rc < 1)
            return DCNV4_ERR_UNSUPPORTED;
    tp->gs_offset = tp->rec_offset + tp->src_cap * p.K * 16;
    tp->splat_lds_bytes = tp->gs_offset + tp->src_cap * tp->gps * 16;
    tp->ctiles_y = (p.H + tp->ch - 1) / tp->ch;
    tp->ctiles_x = (p.W + tp->cw - 1) / tp->cw;
    tp->images_per_launch = (int)(kMaxBytesPerLaunch / image_bytes_max(p, true));
    return DCNV4_OK;
}

// Tile plans depend on the call's geometry only and their search costs up to
// milliseconds on large images, so each distinct geometry is planned once
// and kept (a small cache, oldest entry replaced when full).
class PlanCache {
public:
    int get(const Problem &p, TilePlan *tp, int (*compute)(const Problem &, TilePlan *))
    {
        {
            std::lock_guard<std::mutex> lock(mu_);
            for (const Entry &e : entries_) {
                if (std::memcmp(&e.p, &p, sizeof p) == 0) {
                    *tp = e.plan;
                    return e.status;
                }
            }
        }
        const int st = compute(p, tp);
        std::lock_guard<std::mutex> lock(mu_);
        const Entry e{p, st, *tp};
        if (entries_.size() < kEntries) {
            entries_.push_back(e);
        } else {
            entries_[next_] = e;
            next_ = (next_ + 1) % kEntries;
        }
        return st;
    }

private:
    static constexpr size_t kEntries = 64;
    struct Entry {
        Problem p;
        int status;
        TilePlan plan;
    };
    std::mutex mu_;
    std::vector<Entry> entries_;
    size_t next_ = 0;
};

}  // namespace

int plan_forward_tiled(const Problem &p, TilePlan *tp)
{
    static PlanCache cache;
    return cache.get(p, tp, compute_forward_tiled);
}

int plan_backward_tiled(const Problem &p, TilePlan *tp)
{
    static PlanCache cache;
    return cache.get(p, tp, compute_backward_tiled);
}

}  // namespace dcnv4

namespace dcnv4 {

void clear_hip_error()
{
    g_last_hip_error[0] = '\0';
}

int hip_status(hipError_t e)
{
    if (e == hipSuccess)
        return DCNV4_OK;
    std::snprintf(g_last_hip_error, sizeof g_last_hip_error, "%s: %s", hipGetErrorName(e),
                  hipGetErrorString(e));
    return DCNV4_ERR_HIP;
}

hipError_t allow_dynamic_lds(const void *fn, size_t bytes)
{
    if (bytes <= 64 * 1024)
        return hipSuccess;
    int dev = 0;
    hipError_t e = hipGetDevice(&dev);
    if (e != hipSuccess)
        return e;
    struct Raised {
        const void *fn;
        int dev;
        size_t bytes;
    };
    static std::mutex mu;
    static std::vector<Raised> done;
    std::lock_guard<std::mutex> lock(mu);
    for (const Raised &r : done)
        if (r.fn == fn && r.dev == dev && r.bytes >= bytes)
            return hipSuccess;
    e = hipFuncSetAttribute(fn, hipFuncAttributeMaxDynamicSharedMemorySize, (int)bytes);
    if (e == hipSuccess)
        done.push_back({fn, dev, bytes});
    return e;
}

}  // namespace dcnv4

using namespace dcnv4;

namespace {

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
    const int64_t n = mul_sat(3 * (int64_t)group, K);
    if (n > INT32_MAX)
        return DCNV4_ERR_PARAM;
    const int64_t P = (n + 7) / 8 * 8;
    if (P > INT32_MAX)
        return DCNV4_ERR_PARAM;
    return (int)P;
}

int dcnv4_forward_ex(const void *value, const void *offset_mask, void *output, int N, int H, int W, int kernel_h,
                     int kernel_w, int stride_h, int stride_w, int pad_h, int pad_w, int dilation_h, int dilation_w,
                     int group, int group_channels, float offset_scale, int remove_center, int om_channels,
                     int softmax, int dtype, void *stream)
{
    g_last_hip_error[0] = '\0';
    if (softmax != 0 && softmax != 1)
        return DCNV4_ERR_PARAM;
    Problem p;
    int st = describe(N, H, W, kernel_h, kernel_w, stride_h, stride_w, pad_h, pad_w, dilation_h, dilation_w, group,
                      group_channels, offset_scale, remove_center, om_channels, dtype, &p);
    if (st != DCNV4_OK)
        return st;
    p.softmax = softmax;
    Plan plan;
    TilePlan tp;
    const bool tiled = plan_forward_tiled(p, &tp) == DCNV4_OK;
    st = plan_forward(p, &plan);
    if (softmax && !tiled)
        return DCNV4_ERR_UNSUPPORTED;   // the softmax mode exists in the tiled kernels only
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

int dcnv4_forward(const void *value, const void *offset_mask, void *output, int N, int H, int W, int kernel_h,
                  int kernel_w, int stride_h, int stride_w, int pad_h, int pad_w, int dilation_h, int dilation_w,
                  int group, int group_channels, float offset_scale, int remove_center, int om_channels, int dtype,
                  void *stream)
{
    return dcnv4_forward_ex(value, offset_mask, output, N, H, W, kernel_h, kernel_w, stride_h, stride_w, pad_h, pad_w,
                            dilation_h, dilation_w, group, group_channels, offset_scale, remove_center, om_channels, 0,
                            dtype, stream);
}

int dcnv4_backward_ex(const void *value, const void *offset_mask, const void *grad_output, void *grad_value,
                      void *grad_offset_mask, int N, int H, int W, int kernel_h, int kernel_w, int stride_h,
                      int stride_w, int pad_h, int pad_w, int dilation_h, int dilation_w, int group,
                      int group_channels, float offset_scale, int remove_center, int om_channels, int softmax,
                      int dtype, void *stream)
{
    g_last_hip_error[0] = '\0';
    if (softmax != 0 && softmax != 1)
        return DCNV4_ERR_PARAM;
    Problem p;
    int st = describe(N, H, W, kernel_h, kernel_w, stride_h, stride_w, pad_h, pad_w, dilation_h, dilation_w, group,
                      group_channels, offset_scale, remove_center, om_channels, dtype, &p);
    if (st != DCNV4_OK)
        return st;
    p.softmax = softmax;
    Plan plan;
    TilePlan tp;
    const bool tiled = plan_backward_tiled(p, &tp) == DCNV4_OK;
    st = plan_backward(p, &plan);
    if (softmax && !tiled)
        return DCNV4_ERR_UNSUPPORTED;   // the softmax mode exists in the tiled kernels only
    if (st != DCNV4_OK && !tiled)
        return st;
    if (N == 0)
        return DCNV4_OK;
    if (!value || !offset_mask || !grad_output || !grad_value || !grad_offset_mask)
        return DCNV4_ERR_NULL;
    if (!aligned16(value) || !aligned16(offset_mask) || !aligned16(grad_output) || !aligned16(grad_value) ||
        !aligned16(grad_offset_mask))
        return DCNV4_ERR_ALIGN;
    const int64_t es = p.elem;
    const int64_t img_v = (int64_t)p.H * p.W * p.C * es, img_om = (int64_t)p.Ho * p.Wo * p.P * es,
                  img_o = (int64_t)p.Ho * p.Wo * p.C * es;
    const int64_t img_gv = (int64_t)p.H * p.W * p.C * 4;   // grad_value is fp32 for every dtype
    const int64_t nv = img_v * N, nom = img_om * N, no = img_o * N, ngv = img_gv * N;
    const void *ins[3] = {value, offset_mask, grad_output};
    const int64_t in_sz[3] = {nv, nom, no};
    for (int i = 0; i < 3; ++i) {
        if (ranges_overlap(grad_value, ngv, ins[i], in_sz[i]) ||
            ranges_overlap(grad_offset_mask, nom, ins[i], in_sz[i]))
            return DCNV4_ERR_PARAM;
    }
    if (ranges_overlap(grad_value, ngv, grad_offset_mask, nom))
        return DCNV4_ERR_PARAM;
    hipStream_t s = static_cast<hipStream_t>(stream);
    const int per_launch = tiled ? tp.images_per_launch : plan.images_per_launch;
    for (int n0 = 0; n0 < N; n0 += per_launch) {
        Problem q = p;
        q.N = std::min(per_launch, N - n0);
        const void *v = static_cast<const char *>(value) + img_v * n0;
        const void *om = static_cast<const char *>(offset_mask) + img_om * n0;
        const void *go = static_cast<const char *>(grad_output) + img_o * n0;
        void *gv = static_cast<char *>(grad_value) + img_gv * n0;
        void *gom = static_cast<char *>(grad_offset_mask) + img_om * n0;
        hipError_t e = tiled ? launch_backward_tiled(q, tp, v, om, go, gv, gom, s)
                             : launch_backward_general(q, plan, v, om, go, gv, gom, s);
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
    return dcnv4_backward_ex(value, offset_mask, grad_output, grad_value, grad_offset_mask, N, H, W, kernel_h,
                             kernel_w, stride_h, stride_w, pad_h, pad_w, dilation_h, dilation_w, group,
                             group_channels, offset_scale, remove_center, om_channels, 0, dtype, stream);
}

}  // extern "C"
