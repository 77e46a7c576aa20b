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
                                               const NearSample &s, float m, float (&acc)[DP])
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

// A block owns a th x tw output tile of one (image, group); `lanes` threads
// per pixel, DP channels each.  The value rows of the tile plus a halo of R
// pixels are staged in LDS while each lane loads its pixel's offsets and
// masks into registers; the K samples are unrolled (KMAX >= K).  A far
// sample (rare once R covers the offsets' spread) is taken on the spot from
// global memory.
template <typename T, int DP, int KMAX, bool SM>
__global__ __launch_bounds__(kMaxTileThreads) void dcnv4_fwd_tiled(TArgs a)
{
    extern __shared__ u32x4 smem[];
    constexpr int es = (int)sizeof(T);
    constexpr int NV = DP * es / 16;
    const Geom &geo = a.geo;
    const Tile t = out_tile(a);
    char *val_s = reinterpret_cast<char *>(smem);
    stage_values(a, t, val_s, es);

    const int q = threadIdx.x >> a.lanes_shift;
    const int chunk = threadIdx.x & ((1 << a.lanes_shift) - 1);
    const int py = (int)divm((unsigned)q, a.tw_magic);
    const int px = q - py * a.tw;
    const int oy = t.oy0 + py, ox = t.ox0 + px;
    const bool valid = py < a.th && oy < geo.Ho && ox < geo.Wo;
    OmVectors<T, KMAX> omv;
    omv.load(rsrc(a.om, a.om_bytes),
             valid ? (unsigned)((t.n * geo.Ho + oy) * geo.Wo + ox) * (unsigned)(a.P * es) : kOutOfRange, t.g, a.K);
    staging_done();
    if (!valid)
        return;   // no barrier follows

    float offs[2 * KMAX], msk[KMAX];
    omv.get(offs, msk);
    if (SM) {
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
    const NearFrame nf = near_frame(a, t, oy, ox);
    const char *vb = val_s + chunk * NV * 16;
    const __amdgpu_buffer_rsrc_t vr = rsrc(a.value, a.value_bytes);
    const int chan_off = (t.g * a.Cg + chunk * DP) * es;

    float acc[DP];
#pragma unroll
    for (int c = 0; c < DP; ++c)
        acc[c] = 0.0f;
#pragma unroll
    for (int k = 0; k < KMAX; ++k) {
        if (k < a.K) {
            const float m = msk[k];
            const float bh = nf.bh0 + a.gdh[k], bw = nf.bw0 + a.gdw[k];
            const NearSample s = near_sample(nf, geo.scale, bh, bw, offs[2 * k], offs[2 * k + 1]);
            if (!s.nr && live_loc(geo, s.lh, s.lw))
                far_sample_fwd<T, DP>(geo, vr, t.n, chan_off, s, m, acc);
            // a sample that is not near gets zero weights (its reads hit slot 0)
            const float ah = s.nr ? s.lh - s.fh : 0.0f, aw = s.nr ? s.lw - s.fw : 0.0f;
            const float mm = s.nr ? m : 0.0f;
            const float mh = __builtin_fmaf(-mm, ah, mm), ml = mm * ah;
            const float w00 = __builtin_fmaf(-mh, aw, mh), w01 = mh * aw;
            const float w10 = __builtin_fmaf(-ml, aw, ml), w11 = ml * aw;
            const u32x4 *q00 = reinterpret_cast<const u32x4 *>(vb + s.addr);
            const u32x4 *q01 = reinterpret_cast<const u32x4 *>(vb + s.addr + nf.colb);
            const u32x4 *q10 = reinterpret_cast<const u32x4 *>(vb + s.addr + nf.rowb);
            const u32x4 *q11 = reinterpret_cast<const u32x4 *>(vb + s.addr + nf.rowb + nf.colb);
            u32x4 v00[NV], v01[NV], v10[NV], v11[NV];
#pragma unroll
            for (int v = 0; v < NV; ++v) {
                v00[v] = q00[v];
                v01[v] = q01[v];
                v10[v] = q10[v];
                v11[v] = q11[v];
            }
#pragma unroll
            for (int c = 0; c < DP; ++c) {
                float x = acc[c];
                x = __builtin_fmaf(w00, Store<T>::get(v00, c), x);
                x = __builtin_fmaf(w01, Store<T>::get(v01, c), x);
                x = __builtin_fmaf(w10, Store<T>::get(v10, c), x);
                x = __builtin_fmaf(w11, Store<T>::get(v11, c), x);
                acc[c] = x;
            }
        }
    }

    u32x4 res[NV];
    Store<T>::pack(acc, res, NV);
    u32x4 *dst = reinterpret_cast<u32x4 *>(static_cast<T *>(a.out) +
                                           ((size_t)(t.n * geo.Ho + oy) * geo.Wo + ox) * geo.C + t.g * a.Cg +
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
        return dp == 8 ? fwd_for<_Float16, 8>(small_k, sm) : nullptr;
    case DCNV4_BF16:
        return dp == 8 ? fwd_for<bf16_t, 8>(small_k, sm) : nullptr;
    default:
        return nullptr;
    }
}

}  // namespace tiled
}  // namespace dcnv4
