// LDS-tiled HIP kernels of the DCNv4 spatial aggregation (gfx950 / CDNA4).
//
// Same operation as dcnv4_kernels.hip ("Efficient Deformable ConvNets", CSDN
// walkthrough "DCNv4论文解析", section 1.2 equation without the softmax of
// section 2.1; bilinear sampling with zero padding).
//
// Why tiles: every value element is read ~36 times (9 grid points x 4
// bilinear corners).  The pages rely on on-chip caches and shared memory for
// these re-reads (walkthrough section 2.2; blog "DCNv4架构解析", section
// "并行计算架构设计").  On CDNA4, 128-bit gathers through the texture path
// cost one cache-tag lookup per distinct line and top out near 37 B/clk/CU,
// while random 128-bit LDS reads reach ~77 B/clk/CU when reads are spread
// over all banks.  So a block owns a 2-D tile of output pixels of one (image,
// group), stages the group's value rows of the tile plus a halo of R pixels
// into LDS once (zeros outside the image: the zero-extended image), and
// gathers corners from LDS.  A sample whose integer displacement leaves the
// halo (|floor(loc) - grid position| > R on an axis) is "far" and reads its
// corners from global memory instead.
//
// Backward: device-scope fp32 atomics on this multi-XCD part are resolved
// beyond L2 and LDS fp32 atomics are slow, so grad_value of near samples is
// computed without float atomics: a block owns a tile of *input* cells,
// enumerates the near samples of the output pixels that can reach it, sorts
// their corner contributions by destination cell (a counting sort with
// integer LDS atomics) and sums each cell's list in registers, then writes
// the tile with plain stores.  grad_offset_mask is forward-shaped; it also
// adds the contributions of far samples to grad_value with device atomics,
// after the cell-tile kernel has written every cell.

#include "dcnv4_device.h"
#include "dcnv4_internal.h"

#include <mutex>
#include <utility>
#include <vector>

namespace dcnv4 {
namespace {

using namespace dev;

struct TArgs {
    Geom geo;
    const void *value;
    const void *om;
    void *out;
    const float *gout;
    float *gvalue;
    float *gom;
    int G, Cg, K, P;
    // output tiles
    int th, tw, tiles_y, tiles_x, lanes_shift;
    int R, rh, rw, nvp_shift, swz_mask, swz_shift;
    int om_lds_vecs;             // 16-byte LDS vectors reserved for the offset/mask stage
    int om_dw;                   // staged dwords per pixel (offset/mask entries of one group)
    unsigned k3_magic;           // ceil(2^32 / (3K)): e / (3K) == mulhi(e, k3_magic) for small e
    unsigned tw_magic;           // ceil(2^32 / tw)
    unsigned omdw_magic;         // ceil(2^32 / om_dw)
    unsigned rw_magic;           // ceil(2^32 / rw)
    // cell tiles (backward grad_value)
    int ch, cw, ctiles_y, ctiles_x, src_batch;
    unsigned k_magic;            // ceil(2^32 / K)
    // buffer sizes of this launch, bytes
    int value_bytes, om_bytes, out_bytes, gout_bytes;
};

// e / d for the small non-negative e used here: magic = ceil(2^32 / d), or
// 0 for d = 1 (2^32 does not fit).
__device__ __forceinline__ unsigned divm(unsigned e, unsigned magic)
{
    return magic ? __umulhi(e, magic) : e;
}

// LDS vector slot of vector v of region pixel p.  XOR-ing v with higher
// pixel bits spreads the reads of random pixels over all LDS banks.
__device__ __forceinline__ int vslot(const TArgs &a, int p, int v)
{
    return (p << a.nvp_shift) + (v ^ ((p >> a.swz_shift) & a.swz_mask));
}

struct Tile {
    int n, g, oy0, ox0;
};

// Block -> (image, tile row, tile column, group), group fastest: the groups
// of one tile read the same offset/mask lines and neighbouring value bytes.
__device__ __forceinline__ Tile out_tile(const TArgs &a)
{
    int b = xcd_tile(blockIdx.x, gridDim.x);
    Tile t;
    t.g = b % a.G;
    b /= a.G;
    const int tx = b % a.tiles_x;
    b /= a.tiles_x;
    const int ty = b % a.tiles_y;
    t.n = b / a.tiles_y;
    t.oy0 = ty * a.th;
    t.ox0 = tx * a.tw;
    return t;
}

template <typename T>
__device__ __forceinline__ T load_elem(__amdgpu_buffer_rsrc_t r, unsigned off);
template <>
__device__ __forceinline__ float load_elem<float>(__amdgpu_buffer_rsrc_t r, unsigned off)
{
    return __builtin_bit_cast(float, __builtin_amdgcn_raw_buffer_load_b32(r, off, 0, 0));
}

// Staging uses direct-to-LDS buffer loads: lane t of a wave instruction
// writes its 4 or 16 bytes at LDS base + t*size, a source offset outside the
// buffer writes zeros, and inactive lanes write nothing.  Every wave walks
// contiguous 64-slot chunks of the LDS image, computes the source of each
// slot, and issues all loads before a single wait (the data never passes
// through registers).  Blocks are whole waves (the host rounds the thread
// count up to a multiple of 64; lanes past the tile only help staging).

constexpr unsigned kOutOfRange = 0x80000000u;   // >= any buffer size used here

typedef __attribute__((address_space(3))) void lds_void;

__device__ __forceinline__ void dma16(__amdgpu_buffer_rsrc_t r, void *lds_chunk, unsigned off)
{
    __builtin_amdgcn_raw_ptr_buffer_load_lds(r, (lds_void *)lds_chunk, 16, off, 0, 0, 0);
}

__device__ __forceinline__ void dma4(__amdgpu_buffer_rsrc_t r, void *lds_chunk, unsigned off)
{
    __builtin_amdgcn_raw_ptr_buffer_load_lds(r, (lds_void *)lds_chunk, 4, off, 0, 0, 0);
}

// Offset/mask entries of group g for the tile's pixels, in dwords: pixel q
// owns om_dw dwords starting at dword q*om_dw; they cover its 3K elements
// from the dword-aligned element below g*3K (for 2-byte elements the block's
// entries start om_par elements into each pixel's slice).  Pixels outside the
// image read zeros.
__device__ void stage_offsets(const TArgs &a, const Tile &t, unsigned *om_s, int es)
{
    const Geom &geo = a.geo;
    const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6, nwaves = (blockDim.x + 63) >> 6;
    const int total = a.th * a.tw * a.om_dw;
    const int epd = 4 / es;   // elements per dword
    const __amdgpu_buffer_rsrc_t r = rsrc(a.om, a.om_bytes);
    for (int c0 = wave * 64; c0 < total; c0 += nwaves * 64) {
        const int i = c0 + lane;
        if (i < total) {
            const int q = (int)divm((unsigned)i, a.omdw_magic);
            const int d = i - q * a.om_dw;
            const int py = (int)divm((unsigned)q, a.tw_magic);
            const int px = q - py * a.tw;
            const int oy = t.oy0 + py, ox = t.ox0 + px;
            unsigned off = kOutOfRange;
            if (oy < geo.Ho && ox < geo.Wo) {
                const unsigned e0 = (unsigned)(((t.n * geo.Ho + oy) * geo.Wo + ox) * a.P + t.g * 3 * a.K);
                off = (e0 / (unsigned)epd + (unsigned)d) * 4u;
            }
            dma4(r, om_s + c0, off);
        }
    }
}

// Value rows of group g for the tile plus a halo: region pixel (rr, cc) is
// image pixel (ry0 + rr, rx0 + cc); zeros outside the image.  Slot s holds
// vector (s & (nvp-1)) ^ swizzle(p) of region pixel p = s / nvp (see vslot).
__device__ void stage_region(const TArgs &a, const Tile &t, u32x4 *val_s, int es)
{
    const Geom &geo = a.geo;
    const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6, nwaves = (blockDim.x + 63) >> 6;
    const int ry0 = t.oy0 * geo.sh - geo.ph - a.R, rx0 = t.ox0 * geo.sw - geo.pw - a.R;
    const int total = (a.rh * a.rw) << a.nvp_shift;
    const int vmask = (1 << a.nvp_shift) - 1;
    const unsigned cs = (unsigned)(geo.C * es), goff = (unsigned)(t.g * a.Cg * es);
    const __amdgpu_buffer_rsrc_t vr = rsrc(a.value, a.value_bytes);
    for (int c0 = wave * 64; c0 < total; c0 += nwaves * 64) {
        const int s = c0 + lane;
        if (s < total) {
            const int p = s >> a.nvp_shift;
            const int v = (s & vmask) ^ ((p >> a.swz_shift) & a.swz_mask);
            const int rr = (int)divm((unsigned)p, a.rw_magic);
            const int cc = p - rr * a.rw;
            const int y = ry0 + rr, x = rx0 + cc;
            unsigned off = kOutOfRange;
            if ((unsigned)y < (unsigned)geo.H && (unsigned)x < (unsigned)geo.W)
                off = (unsigned)((t.n * geo.H + y) * geo.W + x) * cs + goff + 16u * (unsigned)v;
            dma16(vr, val_s + c0, off);
        }
    }
}

// Wait for this thread's direct-to-LDS loads, then for the whole block.
__device__ __forceinline__ void staging_done()
{
    __builtin_amdgcn_s_waitcnt(0);
    __syncthreads();
}

// Near test: the integer displacement of the sample is within R pixels.
__device__ __forceinline__ bool near_sample(const Footprint &f, const Loc &l, int R)
{
    return (unsigned)(f.h0 - l.bh + R) <= (unsigned)(2 * R) && (unsigned)(f.w0 - l.bw + R) <= (unsigned)(2 * R);
}

// ---- forward ---------------------------------------------------------------

template <typename T, int DP>
__global__ __launch_bounds__(256) void dcnv4_fwd_tiled(TArgs a)
{
    extern __shared__ u32x4 smem[];
    constexpr int NV = DP * (int)sizeof(T) / 16;
    const Geom &geo = a.geo;
    const Tile t = out_tile(a);
    unsigned *om_s = reinterpret_cast<unsigned *>(smem);
    u32x4 *val_s = smem + a.om_lds_vecs;
    stage_offsets(a, t, om_s, (int)sizeof(T));
    stage_region(a, t, val_s, (int)sizeof(T));
    staging_done();

    const int q = threadIdx.x >> a.lanes_shift;
    const int chunk = threadIdx.x - (q << a.lanes_shift);
    const int py = (int)divm((unsigned)q, a.tw_magic);
    const int px = q - py * a.tw;
    const int oy = t.oy0 + py, ox = t.ox0 + px;
    if (py >= a.th || oy >= geo.Ho || ox >= geo.Wo)
        return;   // no barrier follows
    const int es = (int)sizeof(T);
    constexpr int epd = 4 / (int)sizeof(T);   // elements per staged dword
    const T *om = reinterpret_cast<const T *>(om_s) + q * a.om_dw * epd + ((t.g * 3 * a.K) & (epd - 1));
    const int ry0 = t.oy0 * geo.sh - geo.ph - a.R, rx0 = t.ox0 * geo.sw - geo.pw - a.R;
    const int chan_off = (t.g * a.Cg + chunk * DP) * es;
    const unsigned cs = (unsigned)(geo.C * es), rs = (unsigned)geo.W * cs;
    const __amdgpu_buffer_rsrc_t vr = rsrc(a.value, a.value_bytes);
    const int v0 = chunk * NV;

    float acc[DP];
#pragma unroll
    for (int c = 0; c < DP; ++c)
        acc[c] = 0.0f;

    for (int k = 0; k < a.K; ++k) {
        const float dx = Store<T>::scalar(om[2 * k]);
        const float dy = Store<T>::scalar(om[2 * k + 1]);
        const float m = Store<T>::scalar(om[2 * a.K + k]);
        const Loc l = locate(geo, oy, ox, k, dx, dy);
        if (!live(geo, l))
            continue;
        const Footprint f = footprint(geo, l);
        u32x4 v00[NV], v01[NV], v10[NV], v11[NV];
        float w00, w01, w10, w11;
        if (near_sample(f, l, a.R)) {
            // corners inside the LDS region; outside the image they hold 0
            const float hh = 1.0f - f.lh, hw = 1.0f - f.lw;
            const float mh = m * hh, ml = m * f.lh;
            w00 = mh * hw;
            w01 = mh * f.lw;
            w10 = ml * hw;
            w11 = ml * f.lw;
            const int p00 = (f.h0 - ry0) * a.rw + (f.w0 - rx0);
#pragma unroll
            for (int v = 0; v < NV; ++v) {
                v00[v] = val_s[vslot(a, p00, v0 + v)];
                v01[v] = val_s[vslot(a, p00 + 1, v0 + v)];
                v10[v] = val_s[vslot(a, p00 + a.rw, v0 + v)];
                v11[v] = val_s[vslot(a, p00 + a.rw + 1, v0 + v)];
            }
        } else {
            const unsigned off = corner_offset(geo, t.n, f, es, chan_off);
            masked_weights(f, m, w00, w01, w10, w11);
#pragma unroll
            for (int v = 0; v < NV; ++v) {
                v00[v] = load16(vr, off + 16 * v);
                v01[v] = load16(vr, off + cs + 16 * v);
                v10[v] = load16(vr, off + rs + 16 * v);
                v11[v] = load16(vr, off + rs + cs + 16 * v);
            }
        }
#pragma unroll
        for (int c = 0; c < DP; ++c) {
            float s = acc[c];
            s = __builtin_fmaf(w00, Store<T>::get(v00, c), s);
            s = __builtin_fmaf(w01, Store<T>::get(v01, c), s);
            s = __builtin_fmaf(w10, Store<T>::get(v10, c), s);
            s = __builtin_fmaf(w11, Store<T>::get(v11, c), s);
            acc[c] = s;
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

// ---- backward: grad_offset_mask (and far samples' grad_value) --------------

template <int DP>
__global__ __launch_bounds__(256) void dcnv4_bwd_offsets_tiled(TArgs a)
{
    extern __shared__ u32x4 smem[];
    constexpr int NV = DP / 4;
    const Geom &geo = a.geo;
    const Tile t = out_tile(a);
    float *om_s = reinterpret_cast<float *>(smem);
    u32x4 *val_s = smem + a.om_lds_vecs;
    stage_offsets(a, t, reinterpret_cast<unsigned *>(om_s), 4);
    stage_region(a, t, val_s, 4);
    staging_done();

    const int K3 = 3 * a.K;
    const int q = threadIdx.x >> a.lanes_shift;
    const int chunk = threadIdx.x - (q << a.lanes_shift);
    const int lanes = 1 << a.lanes_shift;
    const int py = (int)divm((unsigned)q, a.tw_magic);
    const int px = q - py * a.tw;
    const int oy = t.oy0 + py, ox = t.ox0 + px;
    // every thread runs the k loop (far samples are written by whole waves);
    // threads past the tile or the image only take part in that
    const bool valid = py < a.th && oy < geo.Ho && ox < geo.Wo;
    float *om = om_s + (valid ? q : 0) * a.om_dw;   // overwritten in place with the gradients
    const int ry0 = t.oy0 * geo.sh - geo.ph - a.R, rx0 = t.ox0 * geo.sw - geo.pw - a.R;
    const int chan_off = (t.g * a.Cg + chunk * DP) * 4;
    const unsigned cs = (unsigned)(geo.C * 4), rs = (unsigned)geo.W * cs;
    const __amdgpu_buffer_rsrc_t vr = rsrc(a.value, a.value_bytes);
    const __amdgpu_buffer_rsrc_t gr = rsrc(a.gvalue, a.value_bytes);
    const __amdgpu_buffer_rsrc_t gor = rsrc(a.gout, a.gout_bytes);
    const int v0 = chunk * NV;
    const unsigned pix_off = ((unsigned)((t.n * geo.Ho + oy) * geo.Wo + ox)) * cs + (unsigned)chan_off;
    // lane's part in a far sample's grad_value update: corner lane / DP,
    // channel lane % DP of the owner's DP channels
    const int lane = threadIdx.x & 63;
    const int my_corner = lane / DP, my_c = lane % DP;
    const unsigned my_corner_off = (unsigned)(my_corner & 1) * cs + (unsigned)(my_corner >> 1) * rs + 4u * (unsigned)my_c;

    float go[DP];
#pragma unroll
    for (int v = 0; v < NV; ++v) {
        const f32x4 r = __builtin_bit_cast(f32x4, load16(gor, valid ? pix_off + 16 * v : kOutOfRange));
        for (int e = 0; e < 4; ++e)
            go[4 * v + e] = r[e];
    }

    for (int k = 0; k < a.K; ++k) {
        const float dx = om[2 * k], dy = om[2 * k + 1], m = om[2 * a.K + k];
        float gm = 0.0f, gw = 0.0f, gh = 0.0f;
        const Loc l = locate(geo, oy, ox, k, dx, dy);
        bool far = false;
        unsigned far_off = 0;
        float w00 = 0.0f, w01 = 0.0f, w10 = 0.0f, w11 = 0.0f;
        if (valid && live(geo, l)) {
            const Footprint f = footprint(geo, l);
            u32x4 v00[NV], v01[NV], v10[NV], v11[NV];
            const bool nr = near_sample(f, l, a.R);
            if (nr) {
                const int p00 = (f.h0 - ry0) * a.rw + (f.w0 - rx0);
#pragma unroll
                for (int v = 0; v < NV; ++v) {
                    v00[v] = val_s[vslot(a, p00, v0 + v)];
                    v01[v] = val_s[vslot(a, p00 + 1, v0 + v)];
                    v10[v] = val_s[vslot(a, p00 + a.rw, v0 + v)];
                    v11[v] = val_s[vslot(a, p00 + a.rw + 1, v0 + v)];
                }
            } else {
                far = true;
                far_off = corner_offset(geo, t.n, f, 4, chan_off);
#pragma unroll
                for (int v = 0; v < NV; ++v) {
                    v00[v] = load16(vr, far_off + 16 * v);
                    v01[v] = load16(vr, far_off + cs + 16 * v);
                    v10[v] = load16(vr, far_off + rs + 16 * v);
                    v11[v] = load16(vr, far_off + rs + cs + 16 * v);
                }
            }
            // t_q = sum_c grad_out_c * v_q,c
            float t00 = 0.0f, t01 = 0.0f, t10 = 0.0f, t11 = 0.0f;
#pragma unroll
            for (int c = 0; c < DP; ++c) {
                t00 = __builtin_fmaf(go[c], Store<float>::get(v00, c), t00);
                t01 = __builtin_fmaf(go[c], Store<float>::get(v01, c), t01);
                t10 = __builtin_fmaf(go[c], Store<float>::get(v10, c), t10);
                t11 = __builtin_fmaf(go[c], Store<float>::get(v11, c), t11);
            }
            if (far) {
                // zero-extended image: dots of corners outside are 0
                t00 = (f.r0 && f.c0) ? t00 : 0.0f;
                t01 = (f.r0 && f.c1) ? t01 : 0.0f;
                t10 = (f.r1 && f.c0) ? t10 : 0.0f;
                t11 = (f.r1 && f.c1) ? t11 : 0.0f;
                masked_weights(f, m, w00, w01, w10, w11);
            }
            const float lh = f.lh, lw = f.lw, hh = 1.0f - lh, hw = 1.0f - lw;
            // d/dm: the sample; d/d loc of the bilinear sample inside the
            // cell chosen by floor (right derivative at integers)
            gm = hh * (hw * t00 + lw * t01) + lh * (hw * t10 + lw * t11);
            gw = hh * (t01 - t00) + lh * (t11 - t10);
            gh = hw * (t10 - t00) + lw * (t11 - t01);
        }
        // grad_value of far samples: one device atomic per corner and
        // channel, issued by the whole wave for one (sample, lane) at a time
        // so that each instruction covers four contiguous corner rows
        unsigned long long fm = __ballot(far);
        while (fm) {
            const int src = __builtin_ctzll(fm);
            fm &= fm - 1;
            const unsigned off = (unsigned)__builtin_amdgcn_readlane((int)far_off, src);
            const float s00 = __builtin_bit_cast(float, __builtin_amdgcn_readlane(__builtin_bit_cast(int, w00), src));
            const float s01 = __builtin_bit_cast(float, __builtin_amdgcn_readlane(__builtin_bit_cast(int, w01), src));
            const float s10 = __builtin_bit_cast(float, __builtin_amdgcn_readlane(__builtin_bit_cast(int, w10), src));
            const float s11 = __builtin_bit_cast(float, __builtin_amdgcn_readlane(__builtin_bit_cast(int, w11), src));
            float g = 0.0f;
#pragma unroll
            for (int c = 0; c < DP; ++c) {
                const float gc = __builtin_bit_cast(float, __builtin_amdgcn_readlane(__builtin_bit_cast(int, go[c]), src));
                g = my_c == c ? gc : g;
            }
            const float w = my_corner == 0 ? s00 : my_corner == 1 ? s01 : my_corner == 2 ? s10 : s11;
            if (my_corner < 4 && w != 0.0f)
                dcnv4_buffer_atomic_fadd(w * g, gr, off + my_corner_off, 0, 0);
        }
        for (int d = 1; d < lanes; d <<= 1) {
            gm += __shfl_xor(gm, d);
            gw += __shfl_xor(gw, d);
            gh += __shfl_xor(gh, d);
        }
        if (valid && chunk == 0) {
            // the lanes of this pixel have read entry k already
            const float sm = geo.scale * m;
            om[2 * k] = sm * gw;
            om[2 * k + 1] = sm * gh;
            om[2 * a.K + k] = gm;
        }
    }
    __syncthreads();

    // write the group's gradient entries of the tile; group 0 also zeroes
    // the padding channels
    {
        const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6, nwaves = (blockDim.x + 63) >> 6;
        const int row_elems = a.tw * K3;
        const __amdgpu_buffer_rsrc_t r = rsrc(a.gom, a.om_bytes);
        const int pad0 = a.G * K3, npad = a.P - pad0;
        for (int py2 = wave; py2 < a.th; py2 += nwaves) {
            const int oy2 = t.oy0 + py2;
            if (oy2 >= geo.Ho)
                break;
            for (int e = lane; e < row_elems; e += 64) {
                const int px2 = (int)divm((unsigned)e, a.k3_magic);
                const int j = e - px2 * K3;
                const int ox2 = t.ox0 + px2;
                if (ox2 < geo.Wo) {
                    const unsigned idx = (unsigned)(((t.n * geo.Ho + oy2) * geo.Wo + ox2) * a.P + t.g * K3 + j);
                    __builtin_amdgcn_raw_buffer_store_b32(__builtin_bit_cast(unsigned, om_s[(py2 * a.tw + px2) * a.om_dw + j]),
                                                          r, idx * 4u, 0, 0);
                }
            }
            if (t.g == 0 && npad > 0) {
                for (int e = lane; e < a.tw * npad; e += 64) {
                    const int px2 = e / npad;
                    const int j = e - px2 * npad;
                    const int ox2 = t.ox0 + px2;
                    if (ox2 < geo.Wo) {
                        const unsigned idx = (unsigned)(((t.n * geo.Ho + oy2) * geo.Wo + ox2) * a.P + pad0 + j);
                        __builtin_amdgcn_raw_buffer_store_b32(0u, r, idx * 4u, 0, 0);
                    }
                }
            }
        }
    }
}

// ---- backward: grad_value of near samples, per cell tile -------------------

constexpr int kSamplesPerLane = 4;   // a batch holds at most 256 * 4 samples
constexpr int kMaxRecords = 4 * 256 * kSamplesPerLane;

__device__ __forceinline__ int floor_div(int a, int b)
{
    const int q = a / b;
    return (a % b != 0 && ((a < 0) != (b < 0))) ? q - 1 : q;
}

__device__ __forceinline__ int ceil_div(int a, int b)
{
    return -floor_div(-a, b);
}

template <int CG>
__global__ __launch_bounds__(256) void dcnv4_bwd_values_tiled(TArgs a)
{
    extern __shared__ u32x4 smem[];
    constexpr int NVG = CG / 4;   // 16-byte vectors of one source pixel's grad_out (fp32)
    const Geom &geo = a.geo;
    unsigned *cnt = reinterpret_cast<unsigned *>(smem);   // [256] records per cell
    unsigned *fill = cnt + 256;                           // [256] scatter cursors
    unsigned *base = fill + 256;                          // [256] exclusive prefix of cnt
    unsigned *wsum = base + 256;                          // [4]  (16 B reserved)
    unsigned *rec = wsum + 4;                             // [2 * kMaxRecords] (weight bits, source)
    u32x4 *g_s = reinterpret_cast<u32x4 *>(rec + 2 * kMaxRecords);   // [src_batch * NVG]

    int b = xcd_tile(blockIdx.x, gridDim.x);
    const int g = b % a.G;
    b /= a.G;
    const int ctx = b % a.ctiles_x;
    b /= a.ctiles_x;
    const int cty = b % a.ctiles_y;
    const int n = b / a.ctiles_y;
    const int cy0 = cty * a.ch, cx0 = ctx * a.cw;
    const int kw = geo.kw;

    // output pixels whose near samples can touch rows [cy0, cy0+ch): a near
    // sample's top row h0 lies in [bh - R, bh + R] with bh = oy*sh - ph + j*dh,
    // and touching needs h0 in [cy0 - 1, cy0 + ch - 1]
    const int sy0 = max(0, ceil_div(cy0 - 1 - a.R + geo.ph - (geo.kh - 1) * geo.dh, geo.sh));
    const int sy1 = min(geo.Ho, floor_div(cy0 + a.ch - 1 + a.R + geo.ph, geo.sh) + 1);
    const int sx0 = max(0, ceil_div(cx0 - 1 - a.R + geo.pw - (kw - 1) * geo.dw, geo.sw));
    const int sx1 = min(geo.Wo, floor_div(cx0 + a.cw - 1 + a.R + geo.pw, geo.sw) + 1);
    const int SW = max(0, sx1 - sx0);
    const int nsrc = max(0, sy1 - sy0) * SW;

    const int tid = threadIdx.x;
    const int lane = tid & 63, wave = tid >> 6;
    const int my_cy = cy0 + tid / a.cw, my_cx = cx0 + tid % a.cw;
    const bool my_cell = tid < a.ch * a.cw;
    const int K3 = 3 * a.K;
    const __amdgpu_buffer_rsrc_t omr = rsrc(a.om, a.om_bytes);
    const __amdgpu_buffer_rsrc_t gor = rsrc(a.gout, a.gout_bytes);
    const unsigned cs = (unsigned)(geo.C * 4);

    float acc[CG];
#pragma unroll
    for (int c = 0; c < CG; ++c)
        acc[c] = 0.0f;

    for (int b0 = 0; b0 < nsrc; b0 += a.src_batch) {
        const int nb = min(a.src_batch, nsrc - b0);
        // (a) grad_out rows of the batch's source pixels
        for (int e = tid; e < nb * NVG; e += 256) {
            const int s = e / NVG, v = e - s * NVG;
            const int src = b0 + s;
            const int oy = sy0 + src / SW, ox = sx0 + src % SW;
            g_s[s * NVG + (v ^ ((s >> a.swz_shift) & a.swz_mask))] =
                load16(gor, (unsigned)((n * geo.Ho + oy) * geo.Wo + ox) * cs + (unsigned)(g * CG * 4 + 16 * v));
        }
        cnt[tid] = 0u;
        fill[tid] = 0u;
        __syncthreads();

        // (b) evaluate this lane's samples; count corner records per cell
        const int ns = nb * a.K;
        unsigned cells[kSamplesPerLane][2];   // four 16-bit cell indices, 0xffff = none
        float wts[kSamplesPerLane][4];
        int srcs[kSamplesPerLane];
#pragma unroll
        for (int i = 0; i < kSamplesPerLane; ++i) {
            cells[i][0] = cells[i][1] = 0xffffffffu;
            const int e = tid + 256 * i;
            srcs[i] = 0;
            if (e < ns) {
                const int s = (int)divm((unsigned)e, a.k_magic);
                const int k = e - s * a.K;
                const int src = b0 + s;
                const int oy = sy0 + src / SW, ox = sx0 + src % SW;
                const unsigned ob = (unsigned)(((n * geo.Ho + oy) * geo.Wo + ox) * a.P + g * K3);
                const float dx = load_elem<float>(omr, (ob + 2 * k) * 4u);
                const float dy = load_elem<float>(omr, (ob + 2 * k + 1) * 4u);
                const float m = load_elem<float>(omr, (ob + 2 * a.K + k) * 4u);
                const Loc l = locate(geo, oy, ox, k, dx, dy);
                if (live(geo, l)) {
                    const Footprint f = footprint(geo, l);
                    if (near_sample(f, l, a.R)) {
                        const float hh = 1.0f - f.lh, hw = 1.0f - f.lw;
                        const float mh = m * hh, ml = m * f.lh;
                        wts[i][0] = mh * hw;
                        wts[i][1] = mh * f.lw;
                        wts[i][2] = ml * hw;
                        wts[i][3] = ml * f.lw;
                        srcs[i] = s;
#pragma unroll
                        for (int qd = 0; qd < 4; ++qd) {
                            const int y = f.h0 + (qd >> 1), x = f.w0 + (qd & 1);
                            const int ly = y - cy0, lx = x - cx0;
                            const bool in = (unsigned)ly < (unsigned)a.ch && (unsigned)lx < (unsigned)a.cw &&
                                            (unsigned)y < (unsigned)geo.H && (unsigned)x < (unsigned)geo.W;
                            if (in) {
                                const unsigned cidx = (unsigned)(ly * a.cw + lx);
                                const int word = qd >> 1, sh = (qd & 1) * 16;
                                cells[i][word] = (cells[i][word] & ~(0xffffu << sh)) | (cidx << sh);
                                atomicAdd(&cnt[cidx], 1u);
                            }
                        }
                    }
                }
            }
        }
        __syncthreads();

        // (c) exclusive prefix sum of the 256 counters
        {
            const unsigned c = cnt[tid];
            unsigned x = c;
            for (int d = 1; d < 64; d <<= 1) {
                const unsigned y = __shfl_up(x, d);
                if (lane >= d)
                    x += y;
            }
            if (lane == 63)
                wsum[wave] = x;
            __syncthreads();
            unsigned off = 0;
            for (int w = 0; w < wave; ++w)
                off += wsum[w];
            base[tid] = off + x - c;
        }
        __syncthreads();

        // (d) scatter (weight, source) records into per-cell lists
#pragma unroll
        for (int i = 0; i < kSamplesPerLane; ++i) {
#pragma unroll
            for (int qd = 0; qd < 4; ++qd) {
                const unsigned cidx = (cells[i][qd >> 1] >> ((qd & 1) * 16)) & 0xffffu;
                if (cidx != 0xffffu) {
                    const unsigned slot = base[cidx] + atomicAdd(&fill[cidx], 1u);
                    rec[2 * slot] = __builtin_bit_cast(unsigned, wts[i][qd]);
                    rec[2 * slot + 1] = (unsigned)srcs[i];
                }
            }
        }
        __syncthreads();

        // (e) each cell sums its list
        if (my_cell) {
            const unsigned r0 = base[tid], r1 = r0 + cnt[tid];
            for (unsigned r = r0; r < r1; ++r) {
                const float w = __builtin_bit_cast(float, rec[2 * r]);
                const int s = (int)rec[2 * r + 1];
#pragma unroll
                for (int v = 0; v < NVG; ++v) {
                    const f32x4 gv = __builtin_bit_cast(f32x4, g_s[s * NVG + (v ^ ((s >> a.swz_shift) & a.swz_mask))]);
                    for (int e2 = 0; e2 < 4; ++e2)
                        acc[4 * v + e2] = __builtin_fmaf(w, gv[e2], acc[4 * v + e2]);
                }
            }
        }
        __syncthreads();
    }

    if (my_cell && my_cy < geo.H && my_cx < geo.W) {
        const __amdgpu_buffer_rsrc_t gvr = rsrc(a.gvalue, a.value_bytes);
        const unsigned off = (unsigned)((n * geo.H + my_cy) * geo.W + my_cx) * cs + (unsigned)(g * CG * 4);
#pragma unroll
        for (int v = 0; v < NVG; ++v) {
            f32x4 o;
            for (int e2 = 0; e2 < 4; ++e2)
                o[e2] = acc[4 * v + e2];
            __builtin_amdgcn_raw_buffer_store_b128(__builtin_bit_cast(u32x4, o), gvr, off + 16 * v, 0, 0);
        }
    }
}

// Launches above 64 KB of dynamic LDS need the kernel's limit raised once
// (gfx950 has 160 KB per CU); remembered per kernel.
hipError_t allow_lds(const void *fn, int bytes)
{
    if (bytes <= 64 * 1024)
        return hipSuccess;
    static std::mutex mu;
    static std::vector<std::pair<const void *, int>> done;
    std::lock_guard<std::mutex> lock(mu);
    for (const auto &d : done)
        if (d.first == fn && d.second >= bytes)
            return hipSuccess;
    const hipError_t e = hipFuncSetAttribute(fn, hipFuncAttributeMaxDynamicSharedMemorySize, bytes);
    if (e == hipSuccess)
        done.emplace_back(fn, bytes);
    return e;
}

unsigned magic_for(int d)
{
    // ceil(2^32 / d): mulhi(e, magic) == e / d for 0 <= e < 2^32 / d;
    // d == 1 is encoded as 0 (see divm)
    if (d == 1)
        return 0u;
    return (unsigned)((((unsigned long long)1 << 32) + (unsigned)d - 1) / (unsigned)d);
}

int log2i(int v)
{
    int s = 0;
    while ((1 << s) < v)
        ++s;
    return s;
}

TArgs make_targs(const Problem &p, const TilePlan &tp)
{
    TArgs a{};
    a.geo = make_geom(p);
    a.G = p.G;
    a.Cg = p.Cg;
    a.K = p.K;
    a.P = p.P;
    a.th = tp.th;
    a.tw = tp.tw;
    a.tiles_y = tp.tiles_y;
    a.tiles_x = tp.tiles_x;
    a.lanes_shift = log2i(tp.lanes);
    a.R = tp.R;
    a.rh = tp.rh;
    a.rw = tp.rw;
    a.nvp_shift = log2i(tp.nvp);
    a.swz_mask = tp.swz_mask;
    a.swz_shift = tp.swz_shift;
    a.om_lds_vecs = tp.om_lds_bytes / 16;
    a.om_dw = tp.om_dw;
    a.k3_magic = magic_for(3 * p.K);
    a.tw_magic = magic_for(tp.tw);
    a.omdw_magic = magic_for(tp.om_dw);
    a.rw_magic = magic_for(tp.rw);
    a.ch = tp.ch;
    a.cw = tp.cw;
    a.ctiles_y = tp.ctiles_y;
    a.ctiles_x = tp.ctiles_x;
    a.src_batch = tp.src_batch;
    a.k_magic = magic_for(p.K);
    return a;
}

}  // namespace

hipError_t launch_forward_tiled(const Problem &p, const TilePlan &tp, const void *value, const void *offset_mask,
                                void *output, hipStream_t stream)
{
    if (tp.threads % 64 != 0 || tp.threads > 256 || tp.threads < tp.th * tp.tw * tp.lanes)
        return hipErrorInvalidConfiguration;
    TArgs a = make_targs(p, tp);
    a.value = value;
    a.om = offset_mask;
    a.out = output;
    a.value_bytes = p.N * p.H * p.W * p.C * p.elem;
    a.om_bytes = p.N * p.Ho * p.Wo * p.P * p.elem;
    a.out_bytes = p.N * p.Ho * p.Wo * p.C * p.elem;
    const int blocks = p.N * tp.tiles_y * tp.tiles_x * p.G;
    const dim3 grid(blocks), block(tp.threads);
#define DCNV4_FWD(T, D)                                                                              \
    do {                                                                                             \
        const hipError_t e_ = allow_lds(reinterpret_cast<const void *>(&dcnv4_fwd_tiled<T, D>), tp.lds_bytes); \
        if (e_ != hipSuccess)                                                                        \
            return e_;                                                                               \
        hipLaunchKernelGGL((dcnv4_fwd_tiled<T, D>), grid, block, tp.lds_bytes, stream, a);           \
    } while (0)
    if (p.dtype == 0) {
        if (tp.dp == 16)
            DCNV4_FWD(float, 16);
        else if (tp.dp == 8)
            DCNV4_FWD(float, 8);
        else if (tp.dp == 4)
            DCNV4_FWD(float, 4);
        else
            return hipErrorInvalidValue;
    } else if (p.dtype == 1) {
        if (tp.dp == 16)
            DCNV4_FWD(_Float16, 16);
        else if (tp.dp == 8)
            DCNV4_FWD(_Float16, 8);
        else
            return hipErrorInvalidValue;
    } else if (p.dtype == 2) {
        if (tp.dp == 16)
            DCNV4_FWD(bf16_t, 16);
        else if (tp.dp == 8)
            DCNV4_FWD(bf16_t, 8);
        else
            return hipErrorInvalidValue;
    } else {
        return hipErrorInvalidValue;
    }
#undef DCNV4_FWD
    return hipGetLastError();
}

hipError_t launch_backward_tiled(const Problem &p, const TilePlan &tp, const void *value, const void *offset_mask,
                                 const void *grad_output, void *grad_value, void *grad_offset_mask,
                                 hipStream_t stream)
{
    if (tp.threads % 64 != 0 || tp.threads > 256 || tp.threads < tp.th * tp.tw * tp.lanes)
        return hipErrorInvalidConfiguration;
    TArgs a = make_targs(p, tp);
    a.value = value;
    a.om = offset_mask;
    a.gout = static_cast<const float *>(grad_output);
    a.gvalue = static_cast<float *>(grad_value);
    a.gom = static_cast<float *>(grad_offset_mask);
    a.value_bytes = p.N * p.H * p.W * p.C * 4;
    a.om_bytes = p.N * p.Ho * p.Wo * p.P * 4;
    a.gout_bytes = p.N * p.Ho * p.Wo * p.C * 4;
    // 1) grad_value of near samples: every cell written once, plain stores
    {
        const int blocks = p.N * tp.ctiles_y * tp.ctiles_x * p.G;
        const dim3 grid(blocks), block(256);
        void (*kern)(TArgs) = nullptr;
        switch (p.Cg) {
        case 4:
            kern = dcnv4_bwd_values_tiled<4>;
            break;
        case 8:
            kern = dcnv4_bwd_values_tiled<8>;
            break;
        case 16:
            kern = dcnv4_bwd_values_tiled<16>;
            break;
        case 32:
            kern = dcnv4_bwd_values_tiled<32>;
            break;
        default:
            return hipErrorInvalidValue;
        }
        hipError_t e = allow_lds(reinterpret_cast<const void *>(kern), tp.splat_lds_bytes);
        if (e != hipSuccess)
            return e;
        hipLaunchKernelGGL(kern, grid, block, tp.splat_lds_bytes, stream, a);
        e = hipGetLastError();
        if (e != hipSuccess)
            return e;
    }
    // 2) grad_offset_mask, plus far samples' grad_value by device atomics
    {
        const int blocks = p.N * tp.tiles_y * tp.tiles_x * p.G;
        const dim3 grid(blocks), block(tp.threads);
        void (*kern)(TArgs) = nullptr;
        switch (tp.dp) {
        case 16:
            kern = dcnv4_bwd_offsets_tiled<16>;
            break;
        case 8:
            kern = dcnv4_bwd_offsets_tiled<8>;
            break;
        case 4:
            kern = dcnv4_bwd_offsets_tiled<4>;
            break;
        default:
            return hipErrorInvalidValue;
        }
        const hipError_t e = allow_lds(reinterpret_cast<const void *>(kern), tp.lds_bytes);
        if (e != hipSuccess)
            return e;
        hipLaunchKernelGGL(kern, grid, block, tp.lds_bytes, stream, a);
    }
    return hipGetLastError();
}

}  // namespace dcnv4
