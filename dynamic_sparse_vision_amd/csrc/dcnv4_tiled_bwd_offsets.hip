// Backward grad_offset_mask kernel of the LDS-tiled DCNv4 path (shared pieces: dcnv4_tiled.h).

#include "dcnv4.h"
#include "dcnv4_tiled.h"

namespace dcnv4 {
namespace tiled {
namespace {

template <typename T, int DP, int KMAX, bool SM>
__global__ __launch_bounds__(kMaxTileThreads) __attribute__((amdgpu_waves_per_eu(KMAX <= 9 ? 4 : 1))) void dcnv4_bwd_offsets_tiled(TArgs a)
{
    extern __shared__ u32x4 smem[];
    constexpr int es = (int)sizeof(T);
    constexpr int NV = DP * es / 16;
    constexpr int EPV = 16 / es;
    constexpr int ES = (3 * KMAX + EPV - 1) / EPV * EPV;   // LDS entries per pixel of the gradient rows
    const Geom &geo = a.geo;
    const Tile t = out_tile(a);
    char *val_s = reinterpret_cast<char *>(smem);
    stage_values(a, t, val_s, es);

    const int q = threadIdx.x >> a.lanes_shift;
    const int chunk = threadIdx.x & ((1 << a.lanes_shift) - 1);
    const int lanes = 1 << a.lanes_shift;
    const int py = (int)divm((unsigned)q, a.tw_magic);
    const int px = q - py * a.tw;
    const int oy = t.oy0 + py, ox = t.ox0 + px;
    // every thread stays to the end (far samples are written by whole waves,
    // and the gradient rows are written back by the block)
    const bool valid = py < a.th && oy < geo.Ho && ox < geo.Wo;
    const unsigned q_pix = (unsigned)((t.n * geo.Ho + oy) * geo.Wo + ox);
    OmVectors<T, KMAX> omv;
    omv.load(rsrc(a.om, a.om_bytes), valid ? q_pix * (unsigned)(a.P * es) : kOutOfRange, t.g, a.K);
    const int chan_off = (t.g * a.Cg + chunk * DP) * es;
    float go[DP];
    {
        const __amdgpu_buffer_rsrc_t gor = rsrc(a.gout, a.gout_bytes);
        u32x4 gv[NV];
#pragma unroll
        for (int v = 0; v < NV; ++v)
            gv[v] = load16(gor, valid ? q_pix * (unsigned)(geo.C * es) + (unsigned)chan_off + 16 * v : kOutOfRange);
#pragma unroll
        for (int c = 0; c < DP; ++c)
            go[c] = Store<T>::get(gv, c);
    }
    staging_done();

    float offs[2 * KMAX], msk[KMAX];
    omv.get(offs, msk);
    if (SM) {
        // msk becomes the probabilities p_k
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
    const unsigned cs = (unsigned)(geo.C * es), rs = (unsigned)geo.W * cs;
    // far samples' grad_value: this lane's part of one atomic instruction
    // (fp32 for every storage dtype): corner lane / DP, channel lane % DP
    const __amdgpu_buffer_rsrc_t gr = rsrc(a.gvalue, a.gvalue_bytes);
    const int lane = threadIdx.x & 63;
    const int my_corner = lane / DP, my_c = lane % DP;
    const unsigned gcs = (unsigned)(geo.C * 4), grs = (unsigned)geo.W * gcs;
    const unsigned my_corner_off = (unsigned)(my_corner & 1) * gcs + (unsigned)(my_corner >> 1) * grs + 4u * (unsigned)my_c;

    // gradients: d/d(dx_k), d/d(dy_k), d/dm_k (d/dp_k in softmax mode until the end)
    float gx[KMAX], gy[KMAX], gmk[KMAX];
#pragma unroll
    for (int k = 0; k < KMAX; ++k) {
        gx[k] = gy[k] = gmk[k] = 0.0f;
        if (k < a.K) {
            const float m = msk[k];
            const float bh = nf.bh0 + a.gdh[k], bw = nf.bw0 + a.gdw[k];
            const NearSample s = near_sample(nf, geo.scale, bh, bw, offs[2 * k], offs[2 * k + 1]);
            const bool nr = s.nr && valid;
            const bool far = valid && !s.nr && live_loc(geo, s.lh, s.lw);
            float t00 = 0.0f, t01 = 0.0f, t10 = 0.0f, t11 = 0.0f;
            unsigned foff = 0;
            float w00 = 0.0f, w01 = 0.0f, w10 = 0.0f, w11 = 0.0f;
            const float ah = s.lh - s.fh, aw = s.lw - s.fw;
            if (far) {
                // corners from global memory; corners outside the image give
                // zero dot products (zero-extended image)
                Footprint f;
                f.h0 = (int)s.fh;
                f.w0 = (int)s.fw;
                f.lh = ah;
                f.lw = aw;
                f.r0 = f.h0 >= 0;
                f.r1 = f.h0 + 1 < geo.H;
                f.c0 = f.w0 >= 0;
                f.c1 = f.w0 + 1 < geo.W;
                foff = corner_offset(geo, t.n, f, es, chan_off);
                u32x4 p00[NV], p01[NV], p10[NV], p11[NV];
                far_corner_loads<NV>(vr, foff, cs, rs, p00, p01, p10, p11);
#pragma unroll
                for (int c = 0; c < DP; ++c) {
                    t00 = __builtin_fmaf(go[c], Store<T>::get(p00, c), t00);
                    t01 = __builtin_fmaf(go[c], Store<T>::get(p01, c), t01);
                    t10 = __builtin_fmaf(go[c], Store<T>::get(p10, c), t10);
                    t11 = __builtin_fmaf(go[c], Store<T>::get(p11, c), t11);
                }
                t00 = (f.r0 && f.c0) ? t00 : 0.0f;
                t01 = (f.r0 && f.c1) ? t01 : 0.0f;
                t10 = (f.r1 && f.c0) ? t10 : 0.0f;
                t11 = (f.r1 && f.c1) ? t11 : 0.0f;
                masked_weights(f, m, w00, w01, w10, w11);
            } else {
                // not near (or no pixel): reads of slot 0, weighted 0 below
                const int addr = nr ? s.addr : 0;
                const u32x4 *q00 = reinterpret_cast<const u32x4 *>(vb + addr);
                const u32x4 *q01 = reinterpret_cast<const u32x4 *>(vb + addr + nf.colb);
                const u32x4 *q10 = reinterpret_cast<const u32x4 *>(vb + addr + nf.rowb);
                const u32x4 *q11 = reinterpret_cast<const u32x4 *>(vb + addr + nf.rowb + nf.colb);
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
                    t00 = __builtin_fmaf(go[c], Store<T>::get(v00, c), t00);
                    t01 = __builtin_fmaf(go[c], Store<T>::get(v01, c), t01);
                    t10 = __builtin_fmaf(go[c], Store<T>::get(v10, c), t10);
                    t11 = __builtin_fmaf(go[c], Store<T>::get(v11, c), t11);
                }
            }
            float gm, gw, gh;
            sample_grads(ah, aw, t00, t01, t10, t11, gm, gw, gh);
            const bool use = nr || far;
            gm = pixel_sum(use ? gm : 0.0f, lanes);
            gw = pixel_sum(use ? gw : 0.0f, lanes);
            gh = pixel_sum(use ? gh : 0.0f, lanes);
            const float sm = geo.scale * m;
            gx[k] = sm * gw;
            gy[k] = sm * gh;
            gmk[k] = gm;
            // grad_value of far samples: the whole wave issues one atomic per
            // (sample, lane), each covering four contiguous corner rows
            unsigned long long fm = __ballot(far);
            while (fm) {
                const int src = __builtin_ctzll(fm);
                fm &= fm - 1;
                // byte offset of the corner in grad_value (fp32) from the
                // value offset (storage dtype; corner_offset wraps consistently)
                const unsigned so = (unsigned)__builtin_amdgcn_readlane((int)foff, src) * (4u / (unsigned)es);
                const float s00 = __builtin_bit_cast(float, __builtin_amdgcn_readlane(__builtin_bit_cast(int, w00), src));
                const float s01 = __builtin_bit_cast(float, __builtin_amdgcn_readlane(__builtin_bit_cast(int, w01), src));
                const float s10 = __builtin_bit_cast(float, __builtin_amdgcn_readlane(__builtin_bit_cast(int, w10), src));
                const float s11 = __builtin_bit_cast(float, __builtin_amdgcn_readlane(__builtin_bit_cast(int, w11), src));
                float g = 0.0f;
#pragma unroll
                for (int c = 0; c < DP; ++c) {
                    const float gc =
                        __builtin_bit_cast(float, __builtin_amdgcn_readlane(__builtin_bit_cast(int, go[c]), src));
                    g = my_c == c ? gc : g;
                }
                const float w = my_corner == 0 ? s00 : my_corner == 1 ? s01 : my_corner == 2 ? s10 : s11;
                if (my_corner < 4 && w != 0.0f)
                    dcnv4_buffer_atomic_fadd(w * g, gr, so + my_corner_off, 0, 0);
            }
        }
    }
    if (SM) {
        // gradients with respect to the logits: p_k * (g_k - sum_j p_j g_j),
        // with g_k = dL/dp_k
        float sdot = 0.0f;
#pragma unroll
        for (int k = 0; k < KMAX; ++k)
            sdot = k < a.K ? __builtin_fmaf(msk[k], gmk[k], sdot) : sdot;
#pragma unroll
        for (int k = 0; k < KMAX; ++k)
            gmk[k] = msk[k] * (gmk[k] - sdot);
    }
    if constexpr (es == 4) {
        // fp32: every entry is dword aligned, so each pixel writes its rows
        // straight from registers with multi-dword stores, no block barrier:
        // the first lane the 2K offsets, the second (or the same) the K masks;
        // group 0 also zeroes the padding channels
        const __amdgpu_buffer_rsrc_t r = rsrc(a.gom, a.om_bytes);
        const unsigned row = q_pix * (unsigned)(a.P * 4);
        const unsigned base = row + (unsigned)(t.g * 3 * a.K * 4);
        const int mask_lane = lanes > 1 ? 1 : 0;
        if (valid && chunk == 0) {
#pragma unroll
            for (int k = 0; k < KMAX; k += 2) {
                if (k + 1 < a.K) {
                    const f32x4 v{gx[k], gy[k], gx[k + 1], gy[k + 1]};
                    __builtin_amdgcn_raw_buffer_store_b128(__builtin_bit_cast(u32x4, v), r, base + 8 * k, 0, 0);
                } else if (k < a.K) {
                    const f32x2 v{gx[k], gy[k]};
                    __builtin_amdgcn_raw_buffer_store_b64(__builtin_bit_cast(u32x2, v), r, base + 8 * k, 0, 0);
                }
            }
        }
        if (valid && chunk == mask_lane) {
            const unsigned mb = base + (unsigned)(8 * a.K);
#pragma unroll
            for (int k = 0; k < KMAX; k += 4) {
                if (k + 3 < a.K) {
                    const f32x4 v{gmk[k], gmk[k + 1], gmk[k + 2], gmk[k + 3]};
                    __builtin_amdgcn_raw_buffer_store_b128(__builtin_bit_cast(u32x4, v), r, mb + 4 * k, 0, 0);
                } else {
#pragma unroll
                    for (int kk = k; kk < k + 4 && kk < KMAX; ++kk)
                        if (kk < a.K)
                            __builtin_amdgcn_raw_buffer_store_b32(__builtin_bit_cast(unsigned, gmk[kk]), r, mb + 4 * kk, 0,
                                                                  0);
                }
            }
            if (t.g == 0) {
                for (int d = a.G * 3 * a.K; d < a.P; ++d)
                    __builtin_amdgcn_raw_buffer_store_b32(0u, r, row + 4u * (unsigned)d, 0, 0);
            }
        }
        return;
    }
    __syncthreads();   // the value rows are no longer read

    // the tile's gradient rows: pixel q's entries from element q*ES, in the
    // offset_mask layout of its group (2K offsets, then K masks)
    if (valid && chunk == 0) {
        // the 2K offsets as whole vectors (entries past 2K are overwritten
        // by the masks below), then the K masks one by one from entry 2K
        constexpr int NVX = (2 * KMAX + EPV - 1) / EPV;
        float xy[NVX * EPV];
#pragma unroll
        for (int i = 0; i < NVX * EPV; ++i)
            xy[i] = 0.0f;
#pragma unroll
        for (int k = 0; k < KMAX; ++k) {
            xy[2 * k] = gx[k];
            xy[2 * k + 1] = gy[k];
        }
        u32x4 xv[NVX];
        Store<T>::pack(xy, xv, NVX);
        char *row = val_s + (size_t)q * ES * es;
#pragma unroll
        for (int v = 0; v < NVX; ++v)
            reinterpret_cast<u32x4 *>(row)[v] = xv[v];
        T *mrow = reinterpret_cast<T *>(row) + 2 * a.K;
#pragma unroll
        for (int k = 0; k < KMAX; ++k)
            if (k < a.K)
                mrow[k] = Store<T>::make(gmk[k]);
    }
    __syncthreads();

    // write the group's gradient entries of the tile back, element for
    // element (2-byte entries of neighbouring groups may share a dword);
    // group 0 also zeroes the padding channels
    {
        const int wave = threadIdx.x >> 6, nwaves = blockDim.x >> 6;
        const __amdgpu_buffer_rsrc_t r = rsrc(a.gom, a.om_bytes);
        const unsigned row_bytes = (unsigned)(geo.Wo * a.P * es);
        const int row0 = t.n * geo.Ho + t.oy0;
        const int rows = min(a.th, geo.Ho - t.oy0);
        const int K3 = 3 * a.K;
        {
            // slot j of a row: entry j % 3K of tile column j / 3K
            unsigned lo[kMaxRowChunks];
            int li[kMaxRowChunks];
            const int row_slots = a.tw * K3;
#pragma unroll
            for (int c = 0; c < kMaxRowChunks; ++c) {
                const int j = c * 64 + lane;
                const int px2 = (int)divm((unsigned)j, a.k3_magic);
                const int d = j - px2 * K3;
                const int ox2 = t.ox0 + px2;
                li[c] = px2 * ES + d;
                lo[c] = (px2 < a.tw && ox2 < geo.Wo) ? (unsigned)((ox2 * a.P + t.g * K3 + d) * es) : kOutOfRange;
            }
            for (int rr = wave; rr < rows; rr += nwaves) {
                const unsigned base = (unsigned)(row0 + rr) * row_bytes;
                const T *src = reinterpret_cast<const T *>(val_s + (size_t)rr * a.tw * ES * es);
#pragma unroll
                for (int c = 0; c < kMaxRowChunks; ++c) {
                    if (c * 64 < row_slots && c * 64 + lane < row_slots && lo[c] != kOutOfRange) {
                        if constexpr (es == 4)
                            __builtin_amdgcn_raw_buffer_store_b32(__builtin_bit_cast(unsigned, src[li[c]]), r,
                                                                  base + lo[c], 0, 0);
                        else
                            __builtin_amdgcn_raw_buffer_store_b16(__builtin_bit_cast(unsigned short, src[li[c]]), r,
                                                                  base + lo[c], 0, 0);
                    }
                }
            }
        }
        const int npad = a.P - a.G * K3;
        if (t.g == 0 && npad > 0) {
            unsigned lo[kMaxRowChunks];
            const int row_slots = a.tw * npad;
#pragma unroll
            for (int c = 0; c < kMaxRowChunks; ++c) {
                const int j = c * 64 + lane;
                const int px2 = (int)divm((unsigned)j, a.npad_magic);
                const int d = j - px2 * npad;
                const int ox2 = t.ox0 + px2;
                lo[c] = (px2 < a.tw && ox2 < geo.Wo) ? (unsigned)((ox2 * a.P + a.G * K3 + d) * es) : kOutOfRange;
            }
            for (int rr = wave; rr < rows; rr += nwaves) {
                const unsigned base = (unsigned)(row0 + rr) * row_bytes;
#pragma unroll
                for (int c = 0; c < kMaxRowChunks; ++c) {
                    if (c * 64 < row_slots && c * 64 + lane < row_slots && lo[c] != kOutOfRange) {
                        if constexpr (es == 4)
                            __builtin_amdgcn_raw_buffer_store_b32(0u, r, base + lo[c], 0, 0);
                        else
                            __builtin_amdgcn_raw_buffer_store_b16((unsigned short)0, r, base + lo[c], 0, 0);
                    }
                }
            }
        }
    }
}


}  // namespace

namespace {

template <typename T, int DP>
Kernel offsets_for(bool small_k, bool sm)
{
    if (small_k)
        return sm ? dcnv4_bwd_offsets_tiled<T, DP, 9, true> : dcnv4_bwd_offsets_tiled<T, DP, 9, false>;
    return sm ? dcnv4_bwd_offsets_tiled<T, DP, 25, true> : dcnv4_bwd_offsets_tiled<T, DP, 25, false>;
}

}  // namespace

Kernel bwd_offsets_kernel(int dtype, int dp, bool small_k, bool sm)
{
    switch (dtype) {
    case DCNV4_FP32:
        return dp == 8 ? offsets_for<float, 8>(small_k, sm) : dp == 4 ? offsets_for<float, 4>(small_k, sm) : nullptr;
    case DCNV4_FP16:
        return dp == 8 ? offsets_for<_Float16, 8>(small_k, sm) : nullptr;
    case DCNV4_BF16:
        return dp == 8 ? offsets_for<bf16_t, 8>(small_k, sm) : nullptr;
    default:
        return nullptr;
    }
}

}  // namespace tiled
}  // namespace dcnv4
