// Backward grad_value (cell-tile) kernel of the LDS-tiled DCNv4 path (shared pieces: dcnv4_tiled.h).

#include "dcnv4.h"
#include "dcnv4_tiled.h"

namespace dcnv4 {
namespace tiled {
namespace {

template <typename T, int CG, int KMAX, bool SM>
__global__ __launch_bounds__(kCellThreads) __attribute__((amdgpu_waves_per_eu(KMAX <= 9 && CG <= 16 ? 4 : 1))) void dcnv4_bwd_values_tiled(TArgs a)
{
    extern __shared__ u32x4 smem[];
    constexpr int es = (int)sizeof(T);
    constexpr int EPV = 16 / es;                           // entries per 16-byte vector
    constexpr int NVG = CG * es / 16;                      // vectors of one source pixel's grad_out
    constexpr int NVO = (2 * KMAX + 2 * (EPV - 1)) / EPV;  // vectors holding the 2K offsets after a shift
    constexpr int NVM = (KMAX + 2 * (EPV - 1)) / EPV;      // vectors holding the K masks after a shift
    const Geom &geo = a.geo;
    char *lds = reinterpret_cast<char *>(smem);
    // [kCellBinSlots]: per-bin counts, then their exclusive prefix in place,
    // then (after placing) the end of each bin
    unsigned *bins = reinterpret_cast<unsigned *>(lds);
    unsigned *wsum = bins + kCellBinSlots;               // [kCellThreads / 64] per-wave scan totals
    // sorted records: (m * (1 - frac h), m * frac h, frac w, LDS byte offset of the
    // source's grad_out)
    f32x4 *rec = reinterpret_cast<f32x4 *>(lds + a.rec_offset);

    int b = xcd_tile(blockIdx.x, gridDim.x);
    const int g = b % a.G;
    b /= a.G;
    const int ctx = b % a.ctiles_x;
    b /= a.ctiles_x;
    const int cty = b % a.ctiles_y;
    const int n = b / a.ctiles_y;
    const int cy0 = cty * a.ch, cx0 = ctx * a.cw;

    // output pixels whose near samples can touch rows [cy0, cy0+ch): a near
    // sample's top row h0 lies in [bh - Rc, bh + Rc] with bh = oy*sh - ph + j*dh,
    // and touching needs h0 in [cy0 - 1, cy0 + ch - 1]
    const int sy0 = max(0, ceil_div(cy0 - 1 - a.Rc + geo.ph - (geo.kh - 1) * geo.dh, geo.sh));
    const int sy1 = min(geo.Ho, floor_div(cy0 + a.ch - 1 + a.Rc + geo.ph, geo.sh) + 1);
    const int sx0 = max(0, ceil_div(cx0 - 1 - a.Rc + geo.pw - (geo.kw - 1) * geo.dw, geo.sw));
    const int sx1 = min(geo.Wo, floor_div(cx0 + a.cw - 1 + a.Rc + geo.pw, geo.sw) + 1);
    const int SW = sx1 - sx0;

    const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
    const int AW = a.cw + 1, NB = (a.ch + 1) * AW;
    // this thread's source within a batch of BR whole source rows
    const int BR = SW > 0 ? max(1, a.src_cap / SW) : 1;
    const int srow = SW > 0 ? tid / SW : 0, scol = tid - srow * SW;
    const int sy_end = SW > 0 ? sy1 : sy0;   // no source column: no batch
    // this thread's pair of cells
    const int py = (int)divm((unsigned)tid, a.cw_magic), px = tid - py * a.cw;
    const bool my_pair = tid < (a.ch >> 1) * a.cw;
    const int binA = 2 * py * AW + px;   // bin row 2py, column px

    const unsigned cs = (unsigned)(geo.C * es);
    const __amdgpu_buffer_rsrc_t omr = rsrc(a.om, a.om_bytes);
    const __amdgpu_buffer_rsrc_t gor = rsrc(a.gout, a.gout_bytes);
    char *g_s = lds + a.gs_offset;   // grad_out of the batch's sources
    const int grow_slots = SW * a.gps;
    // a source's offsets and masks: 16-byte aligned vectors from the one that
    // holds the first entry (pixel rows are 16-byte multiples)
    const int eo = g * 3 * a.K, em = eo + 2 * a.K;
    const int mis_o = eo & (EPV - 1), mis_m = em & (EPV - 1);
    const unsigned vo = (unsigned)((eo - mis_o) * es), vm = (unsigned)((em - mis_m) * es);
    const float Rf = (float)a.Rc, chf = (float)a.ch, cwf = (float)a.cw;
    const float ylo = (float)(cy0 - 1), xlo = (float)(cx0 - 1);
    // LDS byte offset of this thread's source in the staged grad_out
    const unsigned my_gs = (unsigned)a.gs_offset + (unsigned)tid * (unsigned)(a.gps * 16);

    float acc0[CG], acc1[CG];
#pragma unroll
    for (int c = 0; c < CG; ++c)
        acc0[c] = acc1[c] = 0.0f;

    // batch b takes source rows sy0 + b, sy0 + b + nb, ...: every batch
    // spreads its samples over the whole tile, so the waves of a block get
    // similar shares of each batch's gather
    const int SH = sy_end - sy0;
    const int nb = (SH + BR - 1) / BR;
    for (int bt = 0; bt < nb; ++bt) {
        const int r0 = sy0 + bt;
        const int nrows = (SH - bt + nb - 1) / nb;
        for (int i = 4 * tid; i <= NB; i += 4 * kCellThreads)
            *reinterpret_cast<u32x4 *>(bins + i) = u32x4{0u, 0u, 0u, 0u};
        {
            // grad_out rows: slot j of a row is vector j % gps of source
            // column j / gps (offsets made per batch: fewer live registers)
            unsigned glo[kMaxRowChunks];
#pragma unroll
            for (int c = 0; c < kMaxRowChunks; ++c) {
                glo[c] = kOutOfRange;
                if (c * 64 < grow_slots) {
                    const int j = c * 64 + lane;
                    const int s = (int)divm((unsigned)j, a.gps_magic);
                    const int v = j - s * a.gps;
                    if (s < SW && v < NVG)
                        glo[c] = (unsigned)(sx0 + s) * cs + (unsigned)(g * CG * es + 16 * v);
                }
            }
            const unsigned row_bytes = (unsigned)geo.Wo * cs;
            stage_rows<16>(gor, g_s, nrows, grow_slots, glo,
                           [&](int rr) { return (unsigned)(n * geo.Ho + r0 + rr * nb) * row_bytes; });
        }
        const bool src_ok = srow < nrows;
        const int oy = r0 + srow * nb, ox = sx0 + scol;
        const unsigned pix = (unsigned)((n * geo.Ho + oy) * geo.Wo + ox) * (unsigned)(a.P * es);
        u32x4 vov[NVO], vmv[NVM];
#pragma unroll
        for (int j = 0; j < NVO; ++j)
            vov[j] = load16(omr, src_ok ? pix + vo + 16u * j : kOutOfRange);
#pragma unroll
        for (int j = 0; j < NVM; ++j)
            vmv[j] = load16(omr, src_ok ? pix + vm + 16u * j : kOutOfRange);
        staging_done();   // also orders the bin reset before the counting

        float offs[2 * KMAX], msk[KMAX];
        entries_of<T>(vov, mis_o, offs);
        entries_of<T>(vmv, mis_m, msk);
        const float bh0 = (float)(oy * geo.sh - geo.ph), bw0 = (float)(ox * geo.sw - geo.pw);
        // The batch's near samples whose top-left corner cell is in the tile:
        // their bin (relative to (cy0 - 1, cx0 - 1)) and fractional parts.
        // Evaluated twice, to count and then to place, so that nothing but the
        // offsets and masks stays live across the scan.
        auto sample = [&](int k, unsigned &bin, float &fa, float &fb) {
            const float bh = bh0 + a.gdh[k], bw = bw0 + a.gdw[k];
            const float lh = __builtin_fmaf(geo.scale, offs[2 * k + 1], bh);
            const float lw = __builtin_fmaf(geo.scale, offs[2 * k], bw);
            const float fh = __builtin_floorf(lh), fw = __builtin_floorf(lw);
            const bool nr = __builtin_fabsf(fh - bh) <= Rf && __builtin_fabsf(fw - bw) <= Rf;
            const float ay = fh - ylo, ax = fw - xlo;
            fa = lh - fh;
            fb = lw - fw;
            const bool in = src_ok && nr && ay >= 0.0f && ay <= chf && ax >= 0.0f && ax <= cwf;
            // only in-tile floors (small non-negative integers) are converted
            const float cy = in ? ay : 0.0f, cx = in ? ax : 0.0f;
            bin = in ? (unsigned)((int)cy * AW + (int)cx) : 0xffffffffu;
        };
#pragma unroll
        for (int k = 0; k < KMAX; ++k) {
            if (k < a.K) {
                unsigned bin;
                float fa, fb;
                sample(k, bin, fa, fb);
                if (bin != 0xffffffffu)
                    __hip_atomic_fetch_add(&bins[bin], 1u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_WORKGROUP);
            }
        }
        __syncthreads();

        // exclusive prefix of the counts, in place, four bins per thread
        // (entries past NB are not touched)
        {
            const int i0 = 4 * tid;
            u32x4 c = i0 <= NB ? *reinterpret_cast<const u32x4 *>(bins + i0) : u32x4{0u, 0u, 0u, 0u};
            c[1] = i0 + 1 <= NB ? c[1] : 0u;
            c[2] = i0 + 2 <= NB ? c[2] : 0u;
            c[3] = i0 + 3 <= NB ? c[3] : 0u;
            const unsigned mine = c[0] + c[1] + c[2] + c[3];
            const unsigned x = wave_inclusive_sum(mine);
            if (lane == 63)
                wsum[wave] = x;
            __syncthreads();
            unsigned off = 0;
            for (int w = 0; w < wave; ++w)
                off += wsum[w];
            const unsigned e0 = off + x - mine;
            if (i0 <= NB)
                bins[i0] = e0;
            if (i0 + 1 <= NB)
                bins[i0 + 1] = e0 + c[0];
            if (i0 + 2 <= NB)
                bins[i0 + 2] = e0 + c[0] + c[1];
            if (i0 + 3 <= NB)
                bins[i0 + 3] = e0 + c[0] + c[1] + c[2];
        }
        __syncthreads();

        // place the records; afterwards bins[b] is the end of bin b (the
        // start of bin b + 1).  The empty asm hides that the inputs are the
        // same as in the counting pass, so the samples are evaluated again
        // instead of being kept in registers across the scan.
#pragma unroll
        for (int k = 0; k < 2 * KMAX; ++k)
            asm volatile("" : "+v"(offs[k]));
        if (SM) {
            // softmax mode: the records carry the probabilities.  Formed only
            // now, so that logits and probabilities are never live together
            // with the counting pass's values.
            float mx = msk[0];
#pragma unroll
            for (int k = 1; k < KMAX; ++k)
                mx = k < a.K ? fmaxf(mx, msk[k]) : mx;
            float sum = 0.0f;
#pragma unroll
            for (int k = 0; k < KMAX; ++k) {
                msk[k] = k < a.K ? expf(msk[k] - mx) : 0.0f;
                sum += msk[k];
            }
            const float inv = 1.0f / sum;
#pragma unroll
            for (int k = 0; k < KMAX; ++k)
                msk[k] *= inv;
        }
#pragma unroll
        for (int k = 0; k < KMAX; ++k) {
            if (k < a.K) {
                unsigned bin;
                float fa, fb;
                sample(k, bin, fa, fb);
                if (bin != 0xffffffffu) {
                    const unsigned idx = atomicAdd(&bins[bin], 1u);
                    // the mask times the weight of the samples' upper and
                    // lower corner rows, the column fraction, the source
                    f32x4 r;
                    r[0] = msk[k] * (1.0f - fa);
                    r[1] = msk[k] * fa;
                    r[2] = fb;
                    r[3] = __builtin_bit_cast(float, my_gs);
                    rec[idx] = r;
                }
            }
        }
        __syncthreads();

        if (my_pair) {
            // one record ahead: the next record's read overlaps this one's
            // grad_out reads (the read past the end stays inside the LDS
            // allocation and is not used)
            auto gather = [&](int bin, auto &&add) {
                const unsigned s = bin > 0 ? bins[bin - 1] : 0u, mid = bins[bin], e = bins[bin + 1];
                f32x4 rv = rec[s];
                for (unsigned idx = s; idx < e; ++idx) {
                    const f32x4 cur = rv;
                    // LDS byte offset of the source's grad_out (whole-vector cast, then index)
                    const unsigned src = __builtin_bit_cast(u32x4, cur)[3];
                    const u32x4 *gp = reinterpret_cast<const u32x4 *>(lds + src);
                    u32x4 gv[NVG];
#pragma unroll
                    for (int v = 0; v < NVG; ++v)
                        gv[v] = gp[v];
                    rv = rec[idx + 1];
                    // column px of the bin pair: this cell is the samples' right column
                    const float wx = idx < mid ? cur[2] : 1.0f - cur[2];
                    add(cur[0] * wx, cur[1] * wx, gv);
                }
            };
            // bin row 2py: the upper cell is the samples' lower row
            // (wu, wl: the sample's weights on its upper and lower corner row
            // in this cell's column)
            gather(binA, [&](float, float wl, const u32x4(&gv)[NVG]) {
#pragma unroll
                for (int c = 0; c < CG; ++c)
                    acc0[c] = __builtin_fmaf(wl, Store<T>::get(gv, c), acc0[c]);
            });
            // bin row 2py+1: upper row of the upper cell, lower row of the lower
            gather(binA + AW, [&](float wu, float wl, const u32x4(&gv)[NVG]) {
#pragma unroll
                for (int c = 0; c < CG; ++c) {
                    const float gc = Store<T>::get(gv, c);
                    acc0[c] = __builtin_fmaf(wu, gc, acc0[c]);
                    acc1[c] = __builtin_fmaf(wl, gc, acc1[c]);
                }
            });
            // bin row 2py+2: the lower cell is the samples' upper row
            gather(binA + 2 * AW, [&](float wu, float, const u32x4(&gv)[NVG]) {
#pragma unroll
                for (int c = 0; c < CG; ++c)
                    acc1[c] = __builtin_fmaf(wu, Store<T>::get(gv, c), acc1[c]);
            });
        }
        __syncthreads();
    }

    if (my_pair) {
        // grad_value is fp32 for every storage dtype
        const __amdgpu_buffer_rsrc_t gvr = rsrc(a.gvalue, a.gvalue_bytes);
        // the pair's position is taken again from the thread index (made
        // opaque, so it is not kept live, or spilled, across the batches)
        int t2 = tid;
        asm volatile("" : "+v"(t2));
        const int py2 = (int)divm((unsigned)t2, a.cw_magic), px2 = t2 - py2 * a.cw;
        const int my_cy = cy0 + 2 * py2, my_cx = cx0 + px2;
        if (my_cx < geo.W) {
            const unsigned off = ((unsigned)((n * geo.H + my_cy) * geo.W + my_cx) * (unsigned)geo.C + (unsigned)(g * CG)) * 4u;
            const unsigned down = (unsigned)geo.W * (unsigned)geo.C * 4u;
            u32x4 o0[CG / 4], o1[CG / 4];
            Store<float>::pack(acc0, o0, CG / 4);
            Store<float>::pack(acc1, o1, CG / 4);
            if (my_cy < geo.H) {
#pragma unroll
                for (int v = 0; v < CG / 4; ++v)
                    __builtin_amdgcn_raw_buffer_store_b128(o0[v], gvr, off + 16 * v, 0, 0);
            }
            if (my_cy + 1 < geo.H) {
#pragma unroll
                for (int v = 0; v < CG / 4; ++v)
                    __builtin_amdgcn_raw_buffer_store_b128(o1[v], gvr, off + down + 16 * v, 0, 0);
            }
        }
    }
}


}  // namespace

namespace {

template <typename T, int CG>
Kernel values_for(bool small_k, bool sm)
{
    if (small_k)
        return sm ? dcnv4_bwd_values_tiled<T, CG, 9, true> : dcnv4_bwd_values_tiled<T, CG, 9, false>;
    return sm ? dcnv4_bwd_values_tiled<T, CG, 25, true> : dcnv4_bwd_values_tiled<T, CG, 25, false>;
}

template <typename T>
Kernel values_for_cg(int cg, bool small_k, bool sm)
{
    switch (cg) {
    case 4:
        if constexpr (sizeof(T) == 4)
            return values_for<T, 4>(small_k, sm);
        return nullptr;
    case 8:
        return values_for<T, 8>(small_k, sm);
    case 16:
        return values_for<T, 16>(small_k, sm);
    case 32:
        return values_for<T, 32>(small_k, sm);
    default:
        return nullptr;
    }
}

}  // namespace

Kernel bwd_values_kernel(int dtype, int cg, bool small_k, bool sm)
{
    switch (dtype) {
    case DCNV4_FP32:
        return values_for_cg<float>(cg, small_k, sm);
    case DCNV4_FP16:
        return values_for_cg<_Float16>(cg, small_k, sm);
    case DCNV4_BF16:
        return values_for_cg<bf16_t>(cg, small_k, sm);
    default:
        return nullptr;
    }
}

}  // namespace tiled
}  // namespace dcnv4
