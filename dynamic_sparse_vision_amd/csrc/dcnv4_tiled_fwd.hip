// Forward kernel of the LDS-tiled DCNv4 path (shared pieces: dcnv4_tiled.h).

#include "dcnv4.h"
#include "dcnv4_tiled.h"

namespace dcnv4 {
namespace tiled {
namespace {

// ---- forward ---------------------------------------------------------------

// Far sample of the forward: corners from global memory, corners outside
// the image weighted 0 (the buffer range check zero-fills reads past the end).
template <typename T, int DP>
__device__ __forceinline__ void far_sample_fwd(const Geom &geo, __amdgpu_buffer_rsrc_t vr, int n, int chan_off,
                                               const SampleLoc &s, float m, float (&acc)[DP])
{
    constexpr int es = (int)sizeof(T);
    constexpr int NV = DP * es / 16;
    Footprint f;
    f.h0 = (int)s.fh;
    f.w0 = (int)s.fw;
    f.lh = s.lh - s.fh;
    f.lw = s.lw - s.fw;
    f.r0 = f.h0 >= 0;
    f.r1 = f.h0 + 1 < geo.H;
    f.c0 = f.w0 >= 0;
    f.c1 = f.w0 + 1 < geo.W;
    float w00, w01, w10, w11;
    masked_weights(f, m, w00, w01, w10, w11);
    const unsigned cs = (unsigned)(geo.C * es), rs = (unsigned)geo.W * cs;
    u32x4 p00[NV], p01[NV], p10[NV], p11[NV];
    far_corner_loads<NV>(vr, corner_offset(geo, n, f, es, chan_off), cs, rs, p00, p01, p10, p11);
#pragma unroll
    for (int c = 0; c < DP; ++c) {
        float x = acc[c];
        x = __builtin_fmaf(w00, Store<T>::get(p00, c), x);
        x = __builtin_fmaf(w01, Store<T>::get(p01, c), x);
        x = __builtin_fmaf(w10, Store<T>::get(p10, c), x);
        x = __builtin_fmaf(w11, Store<T>::get(p11, c), x);
        acc[c] = x;
    }
}

// A block owns a th x tw output tile of one image and gb groups; per pixel,
// gb x `lanes` threads (groups, then channel chunks, fastest), DP channels
// each (one lane per group of a 16-bit pixel of 16 channels), so that a
// wave's loads of offsets and masks and its output stores cover contiguous
// pixel rows.  The region's value rows are staged in LDS while each lane
// loads its pixel's offsets and masks into registers; the K samples are unrolled
// (KMAX >= K) into one straight-line loop: a sample whose 2x2 footprint lies
// in the region ("near", a test against the block's region bounds) reads its
// corners from LDS, any other gets zero weights there and, if it is live, a
// bit in `far`; after the loop the lanes with far samples take them from
// global memory.  Straight-line code lets the compiler overlap one sample's
// LDS reads with another's arithmetic.
#ifndef DCNV4_FWD_PIPE
#define DCNV4_FWD_PIPE 0
#endif
#ifndef DCNV4_FWD_WAVES
#define DCNV4_FWD_WAVES 4
#endif
template <typename T, int DP, int KMAX, bool SM>
__global__ __launch_bounds__(kMaxTileThreads) __attribute__((amdgpu_waves_per_eu(KMAX <= 9 ? DCNV4_FWD_WAVES : 1))) void dcnv4_fwd_tiled(TArgs a)
{
    extern __shared__ u32x4 smem[];
    constexpr int es = (int)sizeof(T);
    constexpr int NV = DP * es / 16;
    const Geom &geo = a.geo;
    const Tile t = block_tile(a);
    const Region rg = tile_region(a, t);
    char *val_s = reinterpret_cast<char *>(smem);
    stage_region(a, t, rg, val_s, es);

    const int per_pixel_shift = a.lanes_shift + a.gb_shift;
    const int q = threadIdx.x >> per_pixel_shift;
    const int r_in = threadIdx.x & ((1 << per_pixel_shift) - 1);
    const int gl = r_in >> a.lanes_shift;   // group within the block
    const int chunk = r_in & ((1 << a.lanes_shift) - 1);
    const int g = t.g + gl;
    const int py = (int)divm((unsigned)q, a.tw_magic);
    const int px = q - py * a.tw;
    const int oy = t.oy0 + py, ox = t.ox0 + px;
    const bool valid = py < a.th && oy < geo.Ho && ox < geo.Wo;
    // this lane's group slice of the pixel's offsets and masks: aligned
    // 16-byte vectors from the one holding its first entry; the shift inside
    // the vectors differs between the groups of a wave, so it is taken with
    // bit masks, not a branch
    constexpr int EPV = 16 / es;
    constexpr int NVO = (2 * KMAX + 2 * (EPV - 1)) / EPV;
    constexpr int NVM = (KMAX + 2 * (EPV - 1)) / EPV;
    const int eo = g * 3 * a.K, em = eo + 2 * a.K;
    const int mis_o = eo & (EPV - 1), mis_m = em & (EPV - 1);
    u32x4 vov[NVO], vmv[NVM];
    {
        const __amdgpu_buffer_rsrc_t omr = rsrc(a.om, a.om_bytes);
        const unsigned pix = valid ? (unsigned)((t.n * geo.Ho + oy) * geo.Wo + ox) * (unsigned)(a.P * es) : kOutOfRange;
        const unsigned bo = (unsigned)((eo - mis_o) * es), bm = (unsigned)((em - mis_m) * es);
#pragma unroll
        for (int j = 0; j < NVO; ++j)
            vov[j] = load16(omr, pix == kOutOfRange ? kOutOfRange : pix + bo + 16u * j);
#pragma unroll
        for (int j = 0; j < NVM; ++j)
            vmv[j] = load16(omr, pix == kOutOfRange ? kOutOfRange : pix + bm + 16u * j);
    }
    // the grid table, uniform: for up to 9 points loaded once, outside the
    // sample loop (25 points would crowd the scalar registers; they are
    // read where used)
    constexpr int KG = KMAX <= 9 ? KMAX : 1;
    float gdh_r[KG], gdw_r[KG];
#pragma unroll
    for (int k = 0; k < KG; ++k) {
        gdh_r[k] = a.gdh[k];
        gdw_r[k] = a.gdw[k];
    }
    auto gdh = [&](int k) { return KMAX <= 9 ? gdh_r[k < KG ? k : 0] : a.gdh[k]; };
    auto gdw = [&](int k) { return KMAX <= 9 ? gdw_r[k < KG ? k : 0] : a.gdw[k]; };
    staging_done();
    if (!valid)
        return;   // no barrier follows

    // offsets and masks (probabilities in softmax mode: exp(m - sm_max) *
    // sm_inv) from the loaded vectors
    float offs[2 * KMAX], msk[KMAX];
    entries_of<T>(vov, mis_o, offs);
    entries_of<T>(vmv, mis_m, msk);
    float sm_max = 0.0f, sm_inv = 1.0f;
    if (SM) {
        sm_max = msk[0];
#pragma unroll
        for (int k = 1; k < KMAX; ++k)
            sm_max = k < a.K ? fmaxf(sm_max, msk[k]) : sm_max;
        float sum = 0.0f;
#pragma unroll
        for (int k = 0; k < KMAX; ++k) {
            msk[k] = k < a.K ? expf(msk[k] - sm_max) : 0.0f;
            sum += msk[k];
        }
        sm_inv = 1.0f / sum;
#pragma unroll
        for (int k = 0; k < KMAX; ++k)
            msk[k] *= sm_inv;
    }
    const float bh0 = (float)(oy * geo.sh - geo.ph), bw0 = (float)(ox * geo.sw - geo.pw);
    // footprints (fh, fw) .. (fh + 1, fw + 1) inside the region
    const float lo_h = (float)rg.y0, hi_h = (float)(rg.y0 + rg.rows - 2);
    const float lo_w = (float)rg.x0, hi_w = (float)(rg.x0 + rg.cols - 2);
    const unsigned colb = (unsigned)a.pst * 16u, rowb = (unsigned)a.rw * colb;
    const unsigned abias = 0u - (unsigned)rg.y0 * rowb - (unsigned)rg.x0 * colb - (1u << 22) * (rowb + colb);
    // this lane's vectors inside a pixel's slice
    const char *vb = val_s + (gl * a.nvp + chunk * NV) * 16;
    const float Hf = (float)geo.H, Wf = (float)geo.W;

    float acc[DP];
#pragma unroll
    for (int c = 0; c < DP; ++c)
        acc[c] = 0.0f;
    unsigned far = 0;
    // One sample: its placement (near test, weights with the mask folded
    // in, LDS address) and the loads of its four corners.  No branch: points
    // k >= K (KMAX > K) are neither near nor far, and a sample that is not
    // near reads slot 0 with zero weights.
    struct Fetched {
        float w00, w01, w10, w11;
        u32x4 v00[NV], v01[NV], v10[NV], v11[NV];
    };
    auto fetch = [&](int k, Fetched &f) {
        const bool in_k = k < a.K;
        const float lh = __builtin_fmaf(geo.scale, offs[2 * k + 1], bh0 + gdh(k));
        const float lw = __builtin_fmaf(geo.scale, offs[2 * k], bw0 + gdw(k));
        const float fh = __builtin_floorf(lh), fw = __builtin_floorf(lw);
        // false for NaN; huge and infinite coordinates fail as well
        const bool nr = in_k && fh >= lo_h && fh <= hi_h && fw >= lo_w && fw <= hi_w;
        const bool live = in_k && lh >= -1.0f && lh < Hf && lw >= -1.0f && lw < Wf;
        far |= (!nr && live) ? (1u << k) : 0u;
        // floors become integers by bit pattern (defined for every float;
        // see biased_int)
        const unsigned addr = __umul24(biased_int(fh), rowb) + __umul24(biased_int(fw), colb) + abias;
        const unsigned ad = nr ? addr : 0u;
        const float ah = nr ? lh - fh : 0.0f, aw = nr ? lw - fw : 0.0f;
        const float mm = nr ? msk[k] : 0.0f;
        const float mh = __builtin_fmaf(-mm, ah, mm), ml = mm * ah;
        f.w00 = __builtin_fmaf(-mh, aw, mh);
        f.w01 = mh * aw;
        f.w10 = __builtin_fmaf(-ml, aw, ml);
        f.w11 = ml * aw;
        const u32x4 *q00 = reinterpret_cast<const u32x4 *>(vb + ad);
        const u32x4 *q01 = reinterpret_cast<const u32x4 *>(vb + ad + colb);
        const u32x4 *q10 = reinterpret_cast<const u32x4 *>(vb + ad + rowb);
        const u32x4 *q11 = reinterpret_cast<const u32x4 *>(vb + ad + rowb + colb);
#pragma unroll
        for (int v = 0; v < NV; ++v) {
            f.v00[v] = q00[v];
            f.v01[v] = q01[v];
            f.v10[v] = q10[v];
            f.v11[v] = q11[v];
        }
    };
    auto accumulate = [&](const Fetched &f) {
#pragma unroll
        for (int c = 0; c < DP; ++c) {
            float x = acc[c];
            x = __builtin_fmaf(f.w00, Store<T>::get(f.v00, c), x);
            x = __builtin_fmaf(f.w01, Store<T>::get(f.v01, c), x);
            x = __builtin_fmaf(f.w10, Store<T>::get(f.v10, c), x);
            x = __builtin_fmaf(f.w11, Store<T>::get(f.v11, c), x);
            acc[c] = x;
        }
    };
    // Keeps the code in program order around it: the accumulators are
    // complete here (no FMA is deferred past it) and no LDS read moves
    // across it, so at most the reads of one sample ahead are in flight and
    // in registers (left alone, the compiler issues every sample's reads
    // first and runs out of registers).
    // The inputs of sample `next` pass through it as well, so its placement
    // is not computed ahead of the fence either.
    auto fence = [&](int next) {
#pragma unroll
        for (int c = 0; c < DP; ++c)
            asm volatile("" : "+v"(acc[c])::"memory");
        if (next < KMAX)
            asm volatile("" : "+v"(offs[2 * next]), "+v"(offs[2 * next + 1]), "+v"(msk[next]));
    };
    if constexpr (DCNV4_FWD_PIPE == 0) {
        // one sample at a time
#pragma unroll
        for (int k = 0; k < KMAX; ++k) {
            Fetched f;
            fetch(k, f);
            accumulate(f);
            fence(k + 1);
        }
    } else {
        // the next sample's corners are read while this one's are summed
        Fetched f[2];
        fetch(0, f[0]);
        fence(1);
#pragma unroll
        for (int k = 0; k < KMAX; ++k) {
            if (k + 1 < KMAX)
                fetch(k + 1, f[(k + 1) & 1]);
            accumulate(f[k & 1]);
            fence(k + 2);
        }
    }
    if (far) {
        // live samples beyond the region: corners from global memory.  A far
        // sample's offsets and mask are loaded again, one by one (rare; so
        // the entries need not stay in registers through the main loop, and
        // no register array is indexed by a run-time k).
        const __amdgpu_buffer_rsrc_t omr = rsrc(a.om, a.om_bytes);
        const unsigned row = (unsigned)((t.n * geo.Ho + oy) * geo.Wo + ox) * (unsigned)(a.P * es) +
                             (unsigned)(g * 3 * a.K * es);
        auto entry = [&](int idx) -> float {
            if constexpr (es == 4)
                return __builtin_bit_cast(float, __builtin_amdgcn_raw_buffer_load_b32(omr, row + 4u * (unsigned)idx, 0, 0));
            else
                return Store<T>::from_bits(__builtin_amdgcn_raw_buffer_load_b16(omr, row + 2u * (unsigned)idx, 0, 0));
        };
        const __amdgpu_buffer_rsrc_t vr = rsrc(a.value, a.value_bytes);
        const int chan_off = (g * a.Cg + chunk * DP) * es;
        while (far) {
            const int k = __builtin_ctz(far);
            far &= far - 1;
            const float dx = entry(2 * k), dy = entry(2 * k + 1), m0 = entry(2 * a.K + k);
            const float m = SM ? expf(m0 - sm_max) * sm_inv : m0;
            // the grid point from k (a run-time index: no table lookup, which
            // would copy the table to scratch memory)
            int gi, gj;
            grid_point(geo, k, gi, gj);
            SampleLoc s;
            s.lh = __builtin_fmaf(geo.scale, dy, bh0 + (float)(gj * geo.dh));
            s.lw = __builtin_fmaf(geo.scale, dx, bw0 + (float)(gi * geo.dw));
            s.fh = __builtin_floorf(s.lh);
            s.fw = __builtin_floorf(s.lw);
            far_sample_fwd<T, DP>(geo, vr, t.n, chan_off, s, m, acc);
        }
    }

    u32x4 res[NV];
    Store<T>::pack(acc, res, NV);
    u32x4 *dst = reinterpret_cast<u32x4 *>(static_cast<T *>(a.out) +
                                           ((size_t)(t.n * geo.Ho + oy) * geo.Wo + ox) * geo.C + g * a.Cg +
                                           chunk * DP);
#pragma unroll
    for (int v = 0; v < NV; ++v)
        dst[v] = res[v];
}

}  // namespace

namespace {

template <typename T, int DP>
Kernel fwd_for(bool small_k, bool sm)
{
    if (small_k)
        return sm ? dcnv4_fwd_tiled<T, DP, 9, true> : dcnv4_fwd_tiled<T, DP, 9, false>;
    return sm ? dcnv4_fwd_tiled<T, DP, 25, true> : dcnv4_fwd_tiled<T, DP, 25, false>;
}

}  // namespace

Kernel fwd_kernel(int dtype, int dp, bool small_k, bool sm)
{
    switch (dtype) {
    case DCNV4_FP32:
        return dp == 8 ? fwd_for<float, 8>(small_k, sm) : dp == 4 ? fwd_for<float, 4>(small_k, sm) : nullptr;
    case DCNV4_FP16:
        return dp == 16 ? fwd_for<_Float16, 16>(small_k, sm) : dp == 8 ? fwd_for<_Float16, 8>(small_k, sm) : nullptr;
    case DCNV4_BF16:
        return dp == 16 ? fwd_for<bf16_t, 16>(small_k, sm) : dp == 8 ? fwd_for<bf16_t, 8>(small_k, sm) : nullptr;
    default:
        return nullptr;
    }
}

}  // namespace tiled
}  // namespace dcnv4
