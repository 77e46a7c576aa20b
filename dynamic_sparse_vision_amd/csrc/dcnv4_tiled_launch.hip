// Launches of the LDS-tiled DCNv4 kernels: argument packing, the shape
// checks every tiled launch relies on, and the kernel choice by dtype,
// channels per lane (or per group), K bound and mode.

#include "dcnv4.h"
#include "dcnv4_tiled.h"

namespace dcnv4 {

using namespace tiled;

// Shapes every output-tile launch relies on (the planner only produces
// these): gb groups per block (a power of two dividing G), whole waves
// covering the tile's pixels and groups, the region (rh rows of rw pixels at
// an odd stride of gb * nvp slots, at least 2 x 2 pixels) within the block's
// LDS and one staged row within the row chunks.
static bool out_tiles_ok(const Problem &p, const TilePlan &tp)
{
    const int gb = tp.gb;
    return tp.threads % 64 == 0 && tp.threads <= kMaxTileThreads && gb >= 1 && (gb & (gb - 1)) == 0 &&
           p.G % gb == 0 && tp.threads >= tp.th * tp.tw * gb * tp.lanes && p.K <= kMaxTiledPoints &&
           tp.ps == ((gb * tp.nvp) | 1) && tp.rh >= 2 && tp.rw >= 2 && tp.ps * tp.rw <= 64 * kMaxRowChunks &&
           tp.lds_bytes >= tp.rh * tp.rw * tp.ps * 16 && tp.dp * tp.lanes == p.Cg;
}

hipError_t launch_forward_tiled(const Problem &p, const TilePlan &tp, const void *value, const void *offset_mask,
                                void *output, hipStream_t stream)
{
    if (!out_tiles_ok(p, tp))
        return hipErrorInvalidConfiguration;
    const Kernel k = fwd_kernel(p.dtype, tp.dp, p.K <= 9, p.softmax != 0);
    if (!k)
        return hipErrorInvalidValue;
    TArgs a = make_targs(p, tp);
    a.value = value;
    a.om = offset_mask;
    a.out = output;
    a.value_bytes = p.N * p.H * p.W * p.C * p.elem;
    a.om_bytes = p.N * p.Ho * p.Wo * p.P * p.elem;
    a.out_bytes = p.N * p.Ho * p.Wo * p.C * p.elem;
    const int blocks = p.N * tp.tiles_y * tp.tiles_x * (p.G / tp.gb);
    const hipError_t e = allow_dynamic_lds(reinterpret_cast<const void *>(k), (size_t)tp.lds_bytes);
    if (e != hipSuccess)
        return e;
    hipLaunchKernelGGL(k, dim3(blocks), dim3(tp.threads), tp.lds_bytes, stream, a);
    return hipGetLastError();
}

hipError_t launch_backward_tiled(const Problem &p, const TilePlan &tp, const void *value, const void *offset_mask,
                                 const void *grad_output, void *grad_value, void *grad_offset_mask,
                                 hipStream_t stream)
{
    const int es = p.elem;
    if (!out_tiles_ok(p, tp) ||
        // the tile's gradient rows (3K fp32 per pixel and group) reuse the region's LDS
        tp.th * tp.tw * tp.gb * 3 * p.K * 4 > tp.lds_bytes ||
        // grad_value atomics: a power-of-two Cg of at most 64 lanes per corner
        (p.Cg & (p.Cg - 1)) != 0 || p.Cg > 64 || tp.Rc < 0 ||
        // cell tiles
        tp.ch < 2 || tp.ch % 2 != 0 || tp.cw < 1 || (tp.ch / 2) * tp.cw > kCellThreads ||
        (tp.ch + 1) * (tp.cw + 1) >= kCellBinSlots || tp.src_cap < 1 || tp.src_cap > kCellThreads ||
        tp.gps * 16 < p.Cg * es || tp.rec_offset < (kCellBinSlots + kCellThreads / 64) * 4 ||
        tp.rec_offset % 16 != 0 || tp.gs_offset < tp.rec_offset + tp.src_cap * p.K * 16 || tp.gs_offset % 16 != 0 ||
        tp.splat_lds_bytes < tp.gs_offset + tp.src_cap * tp.gps * 16 ||
        // source window width: within a batch and within a staged row
        (tp.cw + 2 * tp.Rc + (p.kw - 1) * p.dw + 1) / p.sw + 2 > tp.src_cap ||
        ((tp.cw + 2 * tp.Rc + (p.kw - 1) * p.dw + 1) / p.sw + 2) * tp.gps > 64 * kMaxRowChunks)
        return hipErrorInvalidConfiguration;
    const bool small_k = p.K <= 9, sm = p.softmax != 0;
    const Kernel values = bwd_values_kernel(p.dtype, p.Cg, small_k, sm);
    const Kernel offsets = bwd_offsets_kernel(p.dtype, tp.dp, small_k, sm);
    if (!values || !offsets)
        return hipErrorInvalidValue;
    TArgs a = make_targs(p, tp);
    a.value = value;
    a.om = offset_mask;
    a.gout = static_cast<const float *>(grad_output);
    a.gvalue = static_cast<float *>(grad_value);
    a.gom = static_cast<float *>(grad_offset_mask);
    a.value_bytes = p.N * p.H * p.W * p.C * es;
    a.om_bytes = p.N * p.Ho * p.Wo * p.P * es;
    a.gout_bytes = p.N * p.Ho * p.Wo * p.C * es;
    a.gvalue_bytes = p.N * p.H * p.W * p.C * 4;
    // 1) grad_value of the samples within Rc: every cell written once, plain stores
    {
        const int blocks = p.N * tp.ctiles_y * tp.ctiles_x * p.G;
        hipError_t e = allow_dynamic_lds(reinterpret_cast<const void *>(values), (size_t)tp.splat_lds_bytes);
        if (e != hipSuccess)
            return e;
        hipLaunchKernelGGL(values, dim3(blocks), dim3(kCellThreads), tp.splat_lds_bytes, stream, a);
        e = hipGetLastError();
        if (e != hipSuccess)
            return e;
    }
    // 2) grad_offset_mask, plus the other samples' grad_value by device atomics
    {
        const int blocks = p.N * tp.tiles_y * tp.tiles_x * (p.G / tp.gb);
        const hipError_t e = allow_dynamic_lds(reinterpret_cast<const void *>(offsets), (size_t)tp.lds_bytes);
        if (e != hipSuccess)
            return e;
        hipLaunchKernelGGL(offsets, dim3(blocks), dim3(tp.threads), tp.lds_bytes, stream, a);
    }
    return hipGetLastError();
}

}  // namespace dcnv4
