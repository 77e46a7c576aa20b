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
// while random 128-bit LDS reads reach ~77 B/clk/CU when a pixel's vectors
// start on an odd 16-byte slot.  So a block owns a 2-D tile of output pixels
// of one (image, group), stages the group's value rows of the tile plus a
// halo of R pixels into LDS once (zeros outside the image: the zero-extended
// image), and gathers corners from LDS.
//
// A sample is "near" when its integer displacement is within R pixels on
// both axes (|floor(loc) - grid position| <= R); its four corners then lie in
// the staged region, so it needs no bounds test at all (corners outside the
// image read the staged zeros).  Other samples are "far" and read their
// corners from global memory where they occur; with R = 7 and offsets of a
// few pixels they are rare.  The R the LDS allows is set by the value rows
// alone: each lane keeps its pixel's offsets and masks in registers.
//
// Staging uses direct-to-LDS buffer loads, one LDS row per group of wave
// instructions: slot j of every row comes from the row's base plus a
// per-lane offset that is the same for all rows, so a slot costs one add.
//
// Backward: device-scope fp32 atomics on this multi-XCD part are resolved
// beyond L2 and LDS fp32 atomics are slow, so grad_value of near samples is
// computed without float atomics: a block owns a tile of *input* cells,
// evaluates the near samples of the output pixels that can reach it, sorts
// them by their top-left corner cell (a counting sort with integer LDS
// atomics), and every thread sums in registers, for a vertical pair of
// cells, the lists of the corner cells that reach them; the tile is then
// written with plain stores.
// grad_offset_mask is forward-shaped; it also adds the contributions of far
// samples to grad_value with device atomics (a whole-wave instruction per far
// sample and lane), after the cell-tile kernel has written every cell.

#include "dcnv4_device.h"
#include "dcnv4_internal.h"

namespace dcnv4 {
namespace {

using namespace dev;

constexpr int kMaxRowChunks = 8;      // a staged row spans at most 8 x 64 slots
constexpr int kMaxTileThreads = 512;  // threads of an output-tile block
constexpr int kMaxTiledPoints = 25;   // K of the tiled kernels (KMAX 9 or 25)
constexpr unsigned kOutOfRange = 0x80000000u;   // >= any buffer size used here

struct TArgs {
    Geom geo;
    const void *value;
    const void *om;
    void *out;
    const float *gout;
    float *gvalue;
    float *gom;
    int G, Cg, K, P;
    // grid point k sits at (j*dh, i*dw) from the window origin (as floats,
    // exact small integers): a table instead of a division by kernel_h
    float gdh[kMaxTiledPoints], gdw[kMaxTiledPoints];
    unsigned k3_magic;           // ceil(2^32 / (3K))
    // output tiles
    int th, tw, tiles_y, tiles_x, lanes_shift;
    int R, rh, rw;               // halo radius; LDS value region, pixels
    int ps, nvp;                 // LDS pixel stride; data vectors per pixel (16-byte units)
    unsigned ps_magic;
    unsigned tw_magic;
    unsigned npad_magic;         // ceil(2^32 / (P - 3GK)), padding entries per pixel
    // cell tiles (backward grad_value)
    int ch, cw, ctiles_y, ctiles_x;
    unsigned cw_magic;           // ceil(2^32 / cw)
    int src_cap;                 // source pixels per batch
    int gps;                     // LDS stride of a staged grad_output pixel, 16-byte units
    unsigned gps_magic;
    int rec_offset, gs_offset;   // LDS byte offsets of the record list and the grad_output rows
    // buffer sizes of this launch, bytes
    int value_bytes, om_bytes, out_bytes, gout_bytes;
    int gvalue_bytes;            // grad_value is fp32 for every storage dtype
};

// e / d for the small non-negative e used here: magic = ceil(2^32 / d), or
// 0 for d = 1 (2^32 does not fit).
__device__ __forceinline__ unsigned divm(unsigned e, unsigned magic)
{
    return magic ? __umulhi(e, magic) : e;
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

// ---- staging ----------------------------------------------------------------

typedef __attribute__((address_space(3))) void lds_void;

// Direct-to-LDS buffer load: lane t of the wave writes its SZ bytes at
// lds + t*SZ; a source offset outside the buffer writes zeros, inactive lanes
// write nothing.
template <int SZ>
__device__ __forceinline__ void dma(__amdgpu_buffer_rsrc_t r, void *lds, unsigned off)
{
    static_assert(SZ == 4 || SZ == 16, "slot size");
    if constexpr (SZ == 4)
        __builtin_amdgcn_raw_ptr_buffer_load_lds(r, (lds_void *)lds, 4, off, 0, 0, 0);
    else
        __builtin_amdgcn_raw_ptr_buffer_load_lds(r, (lds_void *)lds, 16, off, 0, 0, 0);
}

// Copy `nrows` rows of `row_slots` SZ-byte slots into LDS (row rr at slot
// rr*row_slots).  Slot j of row rr is read from row_off(rr) + lane_off[j/64]
// of lane j%64, or is zero when either is kOutOfRange.  Waves take whole rows.
template <int SZ, typename RowOff>
__device__ __forceinline__ void stage_rows(__amdgpu_buffer_rsrc_t r, char *lds, int nrows, int row_slots,
                                           const unsigned (&lane_off)[kMaxRowChunks], RowOff row_off)
{
    const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6, nwaves = blockDim.x >> 6;
    for (int rr = wave; rr < nrows; rr += nwaves) {
        const unsigned base = row_off(rr);
        char *dst = lds + rr * row_slots * SZ;
#pragma unroll
        for (int c = 0; c < kMaxRowChunks; ++c) {
            if (c * 64 < row_slots && c * 64 + lane < row_slots) {
                const unsigned lo = lane_off[c];
                dma<SZ>(r, dst + c * 64 * SZ, (base == kOutOfRange || lo == kOutOfRange) ? kOutOfRange : base + lo);
            }
        }
    }
}

// Wait for this thread's direct-to-LDS and buffer loads, then for the block.
__device__ __forceinline__ void staging_done()
{
    __builtin_amdgcn_s_waitcnt(0);
    __syncthreads();
}

// Value rows of group g for the tile plus the halo: region pixel (rr, cc) is
// image pixel (ry0 + rr, rx0 + cc) and starts at 16-byte slot
// (rr*rw + cc)*ps; zeros outside the image.
__device__ __forceinline__ void stage_values(const TArgs &a, const Tile &t, char *val_s, int es)
{
    const Geom &geo = a.geo;
    const int lane = threadIdx.x & 63;
    {
        unsigned lo[kMaxRowChunks];
        const int row_slots = a.rw * a.ps;
        const int rx0 = t.ox0 * geo.sw - geo.pw - a.R;
        const unsigned cs = (unsigned)(geo.C * es), goff = (unsigned)(t.g * a.Cg * es);
#pragma unroll
        for (int c = 0; c < kMaxRowChunks; ++c) {
            lo[c] = kOutOfRange;
            if (c * 64 < row_slots) {
                const int j = c * 64 + lane;
                const int cc = (int)divm((unsigned)j, a.ps_magic);
                const int v = j - cc * a.ps;
                const int x = rx0 + cc;
                if (v < a.nvp && cc < a.rw && (unsigned)x < (unsigned)geo.W)
                    lo[c] = (unsigned)x * cs + goff + 16u * (unsigned)v;
            }
        }
        const int ry0 = t.oy0 * geo.sh - geo.ph - a.R;
        const unsigned row_bytes = (unsigned)geo.W * cs;
        stage_rows<16>(rsrc(a.value, a.value_bytes), val_s, a.rh, row_slots, lo, [&](int rr) {
            const int y = ry0 + rr;
            return (unsigned)y < (unsigned)geo.H ? (unsigned)(t.n * geo.H + y) * row_bytes : kOutOfRange;
        });
    }
}

// ---- offsets and masks in registers ------------------------------------------
//
// A pixel's group slice of offset_mask starts at the same element offset in
// every pixel row, so its misalignment inside a 16-byte vector (mis) is the
// same for the whole block.  A lane loads the aligned vectors that cover the
// slice, and the shift is a register renaming chosen once per block (a
// switch on mis) rather than per-lane arithmetic.

template <typename T, int NVEC, int NOUT, int MIS>
__device__ __forceinline__ void take_entries(const u32x4 (&v)[NVEC], float (&out)[NOUT])
{
    constexpr int EPV = 16 / (int)sizeof(T);
    static_assert(MIS + NOUT <= EPV * NVEC, "vectors too short");
    // keeps the cases of entries_at apart: merged, they would become one
    // dynamically indexed array in scratch memory
    asm volatile("; entries shifted by %0" ::"n"(MIS));
    unsigned w[4 * NVEC];
#pragma unroll
    for (int i = 0; i < NVEC; ++i)
#pragma unroll
        for (int e = 0; e < 4; ++e)
            w[4 * i + e] = v[i][e];
#pragma unroll
    for (int e = 0; e < NOUT; ++e) {
        const int idx = e + MIS;
        if constexpr (sizeof(T) == 4)
            out[e] = __builtin_bit_cast(float, w[idx]);
        else
            out[e] = Store<T>::from_bits((idx & 1) ? w[idx >> 1] >> 16 : w[idx >> 1]);
    }
}

template <typename T, int NVEC, int NOUT>
__device__ __forceinline__ void entries_at(const u32x4 (&v)[NVEC], int mis, float (&out)[NOUT])
{
    switch (mis) {
    case 0: take_entries<T, NVEC, NOUT, 0>(v, out); break;
    case 1: take_entries<T, NVEC, NOUT, 1>(v, out); break;
    case 2: take_entries<T, NVEC, NOUT, 2>(v, out); break;
    case 3: take_entries<T, NVEC, NOUT, 3>(v, out); break;
    default:
        if constexpr (sizeof(T) == 2) {
            switch (mis) {
            case 4: take_entries<T, NVEC, NOUT, 4>(v, out); break;
            case 5: take_entries<T, NVEC, NOUT, 5>(v, out); break;
            case 6: take_entries<T, NVEC, NOUT, 6>(v, out); break;
            default: take_entries<T, NVEC, NOUT, 7>(v, out); break;
            }
        }
        break;
    }
}

// Vectors covering a pixel's 2K offsets and K masks (group g, entries from
// element g*3K of the pixel's row).
template <typename T, int KMAX>
struct OmVectors {
    static constexpr int EPV = 16 / (int)sizeof(T);
    static constexpr int NVO = (2 * KMAX + 2 * (EPV - 1)) / EPV;
    static constexpr int NVM = (KMAX + 2 * (EPV - 1)) / EPV;
    u32x4 o[NVO], m[NVM];
    int mis_o, mis_m;

    // pix: byte offset of the pixel's row, or kOutOfRange (zeros)
    __device__ __forceinline__ void load(__amdgpu_buffer_rsrc_t r, unsigned pix, int g, int K)
    {
        const int eo = g * 3 * K, em = eo + 2 * K;
        mis_o = eo & (EPV - 1);
        mis_m = em & (EPV - 1);
        const unsigned bo = (unsigned)((eo - mis_o) * (int)sizeof(T)), bm = (unsigned)((em - mis_m) * (int)sizeof(T));
#pragma unroll
        for (int j = 0; j < NVO; ++j)
            o[j] = load16(r, pix == kOutOfRange ? kOutOfRange : pix + bo + 16u * j);
#pragma unroll
        for (int j = 0; j < NVM; ++j)
            m[j] = load16(r, pix == kOutOfRange ? kOutOfRange : pix + bm + 16u * j);
    }

    __device__ __forceinline__ void get(float (&offs)[2 * KMAX], float (&msk)[KMAX]) const
    {
        entries_at<T>(o, mis_o, offs);
        entries_at<T>(m, mis_m, msk);
    }
};

// Per-pixel constants of the near test and of LDS corner addresses.
struct NearFrame {
    float bh0, bw0;   // integer base of grid point (0, 0), as floats
    float Rf;
    int rowb, colb;   // LDS bytes per region row / pixel
    int abase;        // LDS byte address of image pixel (0, 0) relative to the region
};

__device__ __forceinline__ NearFrame near_frame(const TArgs &a, const Tile &t, int oy, int ox)
{
    const Geom &geo = a.geo;
    NearFrame f;
    f.bh0 = (float)(oy * geo.sh - geo.ph);
    f.bw0 = (float)(ox * geo.sw - geo.pw);
    f.Rf = (float)a.R;
    f.colb = a.ps * 16;
    f.rowb = a.rw * f.colb;
    const int ry0 = t.oy0 * geo.sh - geo.ph - a.R, rx0 = t.ox0 * geo.sw - geo.pw - a.R;
    f.abase = -(ry0 * f.rowb + rx0 * f.colb);
    return f;
}

// One sample in the main loops: location, floor, near test (false for NaN),
// and the LDS byte address of the top-left corner when near (0 otherwise).
struct NearSample {
    float lh, lw, fh, fw;
    bool nr;
    int addr;
};

__device__ __forceinline__ NearSample near_sample(const NearFrame &f, float scale, float bh, float bw, float dx,
                                                  float dy)
{
    NearSample s;
    s.lh = __builtin_fmaf(scale, dy, bh);
    s.lw = __builtin_fmaf(scale, dx, bw);
    s.fh = __builtin_floorf(s.lh);
    s.fw = __builtin_floorf(s.lw);
    // fh - bh and fw - bw are differences of integers below 2^24 (or huge)
    s.nr = __builtin_fabsf(s.fh - bh) <= f.Rf && __builtin_fabsf(s.fw - bw) <= f.Rf;
    // near: |fh|, |fw| are below 2^23, so 24-bit multiplies are exact
    const int addr = __mul24((int)s.fh, f.rowb) + __mul24((int)s.fw, f.colb) + f.abase;
    s.addr = s.nr ? addr : 0;
    return s;
}

__device__ __forceinline__ bool live_loc(const Geom &g, float lh, float lw)
{
    return lh >= -1.0f && lh < (float)g.H && lw >= -1.0f && lw < (float)g.W;
}

// Corners of a far sample from global memory: loads only (the caller uses
// the registers later, so the loads overlap other work).
template <int NV>
__device__ __forceinline__ void far_corner_loads(__amdgpu_buffer_rsrc_t vr, unsigned off, unsigned cs, unsigned rs,
                                                 u32x4 (&v00)[NV], u32x4 (&v01)[NV], u32x4 (&v10)[NV],
                                                 u32x4 (&v11)[NV])
{
#pragma unroll
    for (int v = 0; v < NV; ++v) {
        v00[v] = load16(vr, off + 16 * v);
        v01[v] = load16(vr, off + cs + 16 * v);
        v10[v] = load16(vr, off + rs + 16 * v);
        v11[v] = load16(vr, off + rs + cs + 16 * v);
    }
}

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

// ---- backward: grad_offset_mask (and far samples' grad_value) --------------

// Gradients of one sample from the dot products t_q = sum_c grad_out_c *
// v_q,c of its four corners: d/dm is the bilinear sample; d/d loc is the
// derivative inside the cell chosen by floor (right derivative at integers).
__device__ __forceinline__ void sample_grads(float ah, float aw, float t00, float t01, float t10, float t11,
                                             float &gm, float &gw, float &gh)
{
    const float hh = 1.0f - ah, hw = 1.0f - aw;
    gm = hh * __builtin_fmaf(hw, t00, aw * t01) + ah * __builtin_fmaf(hw, t10, aw * t11);
    gw = hh * (t01 - t00) + ah * (t11 - t10);
    gh = hw * (t10 - t00) + aw * (t11 - t01);
}

// Sum of x over the `lanes` consecutive lanes of a pixel (1, 2, 4, ... 64;
// uniform): DPP swaps inside quads, then lane swizzles.
__device__ __forceinline__ float pixel_sum(float x, int lanes)
{
    if (lanes >= 2)
        x += __builtin_bit_cast(float, __builtin_amdgcn_mov_dpp(__builtin_bit_cast(int, x), 0xB1, 0xF, 0xF, false));
    if (lanes >= 4)
        x += __builtin_bit_cast(float, __builtin_amdgcn_mov_dpp(__builtin_bit_cast(int, x), 0x4E, 0xF, 0xF, false));
    for (int d = 4; d < lanes; d <<= 1)
        x += __shfl_xor(x, d);
    return x;
}

// A block owns a th x tw output tile of one (image, group), as in the
// forward.  Per sample the dot products t_q = sum_c grad_out_c * v_q,c of the
// four corners give d/dm and d/d(loc) (right derivative at integers), summed
// over the pixel's lanes; the 3K gradients of a pixel stay in registers (the
// samples are unrolled, KMAX >= K).  A far sample reads its corners from
// global memory on the spot and adds its grad_value contributions with
// device atomics, one 64-lane instruction per (sample, lane) taken by the
// whole wave.  At the end the value rows are no longer needed and their LDS
// holds the tile's gradient rows, which are written back row by row.
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

// ---- backward: grad_value of near samples, per cell tile -------------------

__device__ __forceinline__ int floor_div(int a, int b)
{
    const int q = a / b;
    return (a % b != 0 && ((a < 0) != (b < 0))) ? q - 1 : q;
}

__device__ __forceinline__ int ceil_div(int a, int b)
{
    return -floor_div(-a, b);
}

// Entries e = 0..NOUT-1 of a slice that starts `mis` (0..3, the same for the
// whole block) dwords into the 16-byte vectors v.  The shift is done with
// bit masks, not as an array index (which would go through scratch memory).
template <int NVEC, int NOUT>
__device__ __forceinline__ void shifted_entries(const u32x4 (&v)[NVEC], int mis, float (&out)[NOUT])
{
    static_assert(NOUT + 3 <= 4 * NVEC, "vectors too short");
    unsigned w[4 * NVEC];
#pragma unroll
    for (int i = 0; i < NVEC; ++i)
        for (int e = 0; e < 4; ++e)
            w[4 * i + e] = v[i][e];
    const unsigned m1 = 0u - (unsigned)(mis & 1), m2 = 0u - (unsigned)((mis >> 1) & 1);
    unsigned t[4 * NVEC - 1];
#pragma unroll
    for (int i = 0; i < 4 * NVEC - 1; ++i)
        t[i] = w[i] ^ ((w[i] ^ w[i + 1]) & m1);
#pragma unroll
    for (int e = 0; e < NOUT; ++e)
        out[e] = __builtin_bit_cast(float, t[e] ^ ((t[e] ^ t[e + 2]) & m2));
}

// 2-byte entries e = 0..NOUT-1 of a slice that starts `mis` (0..7, the same
// for the whole block) elements into the 16-byte vectors v, as floats: a
// dword shift by mis / 2, then a half-word select by mis % 2, all with bit
// masks.
template <typename T, int NVEC, int NOUT>
__device__ __forceinline__ void shifted_entries16(const u32x4 (&v)[NVEC], int mis, float (&out)[NOUT])
{
    static_assert(NOUT + 7 <= 8 * NVEC, "vectors too short");
    unsigned w[4 * NVEC];
#pragma unroll
    for (int i = 0; i < NVEC; ++i)
        for (int e = 0; e < 4; ++e)
            w[4 * i + e] = v[i][e];
    const int sh = mis >> 1;
    const unsigned m1 = 0u - (unsigned)(sh & 1), m2 = 0u - (unsigned)((sh >> 1) & 1);
    unsigned t1[4 * NVEC - 1], W[4 * NVEC - 3];
#pragma unroll
    for (int i = 0; i < 4 * NVEC - 1; ++i)
        t1[i] = w[i] ^ ((w[i] ^ w[i + 1]) & m1);
#pragma unroll
    for (int i = 0; i < 4 * NVEC - 3; ++i)
        W[i] = t1[i] ^ ((t1[i] ^ t1[i + 2]) & m2);
    const unsigned mp = 0u - (unsigned)(mis & 1);
#pragma unroll
    for (int e = 0; e < NOUT; ++e) {
        const unsigned even = (e & 1) ? (W[e >> 1] >> 16) : (W[e >> 1] & 0xffffu);
        const unsigned odd = (e & 1) ? (W[(e + 1) >> 1] & 0xffffu) : (W[e >> 1] >> 16);
        out[e] = Store<T>::from_bits(even ^ ((even ^ odd) & mp));
    }
}

template <typename T, int NVEC, int NOUT>
__device__ __forceinline__ void entries_of(const u32x4 (&v)[NVEC], int mis, float (&out)[NOUT])
{
    if constexpr (sizeof(T) == 4)
        shifted_entries(v, mis, out);
    else
        shifted_entries16<T>(v, mis, out);
}

// Inclusive prefix sum over the 64 lanes of a wave with DPP: shifts by 1, 2,
// 4, 8 inside rows of 16 lanes, then lane 15 of rows 0 and 2 added to rows 1
// and 3, then lane 31 to rows 2 and 3 (lanes without a source add 0).
__device__ __forceinline__ unsigned wave_inclusive_sum(unsigned v)
{
    int x = (int)v;
    x += __builtin_amdgcn_update_dpp(0, x, 0x111, 0xF, 0xF, false);   // row_shr:1
    x += __builtin_amdgcn_update_dpp(0, x, 0x112, 0xF, 0xF, false);   // row_shr:2
    x += __builtin_amdgcn_update_dpp(0, x, 0x114, 0xF, 0xF, false);   // row_shr:4
    x += __builtin_amdgcn_update_dpp(0, x, 0x118, 0xF, 0xF, false);   // row_shr:8
    x += __builtin_amdgcn_update_dpp(0, x, 0x142, 0xA, 0xF, false);   // row_bcast:15
    x += __builtin_amdgcn_update_dpp(0, x, 0x143, 0xC, 0xF, false);   // row_bcast:31
    return (unsigned)x;
}

// A cell-tile block: ch x cw input cells of one (image, group), ch even;
// thread t < (ch / 2) * cw owns the vertical pair of cells (2 * (t / cw),
// t % cw) and the one below it.  The output pixels whose near samples can
// reach the tile (its "sources") are taken in batches of whole rows; a batch
// stages their grad_output rows, evaluates their samples (one source per
// thread), and counting-sorts the near samples by top-left corner cell
// ("bin"; bins span rows cy0-1 .. cy0+ch-1 and columns cx0-1 .. cx0+cw-1).
// A sample's corners are the cells of bin rows by, by+1 and columns bx,
// bx+1, so the pair sums three runs of the sorted list: bin row 2py (its
// upper cell is the samples' lower corner row), 2py+1 (both cells) and 2py+2
// (its lower cell is their upper row); each run is the two bins of columns
// px and px+1, which are adjacent in the sorted order.  Every record adds
// to exactly the cells that are its corners (non-finite inputs spread as in
// the plain sum).
template <typename T, int CG, int KMAX, bool SM>
__global__ __launch_bounds__(kCellThreads) __attribute__((amdgpu_waves_per_eu(KMAX <= 9 ? 4 : 1))) void dcnv4_bwd_values_tiled(TArgs a)
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
    // sample's top row h0 lies in [bh - R, bh + R] with bh = oy*sh - ph + j*dh,
    // and touching needs h0 in [cy0 - 1, cy0 + ch - 1]
    const int sy0 = max(0, ceil_div(cy0 - 1 - a.R + geo.ph - (geo.kh - 1) * geo.dh, geo.sh));
    const int sy1 = min(geo.Ho, floor_div(cy0 + a.ch - 1 + a.R + geo.ph, geo.sh) + 1);
    const int sx0 = max(0, ceil_div(cx0 - 1 - a.R + geo.pw - (geo.kw - 1) * geo.dw, geo.sw));
    const int sx1 = min(geo.Wo, floor_div(cx0 + a.cw - 1 + a.R + geo.pw, geo.sw) + 1);
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
    const float Rf = (float)a.R, chf = (float)a.ch, cwf = (float)a.cw;
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
            bin = in ? (unsigned)((int)ay * AW + (int)ax) : 0xffffffffu;
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
        const int my_cy = cy0 + 2 * py, my_cx = cx0 + px;
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

unsigned magic_for(int d)
{
    // ceil(2^32 / d): mulhi(e, magic) == e / d for 0 <= e < 2^32 / d;
    // d == 1 is encoded as 0 (see divm)
    if (d <= 1)
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
    a.k3_magic = magic_for(3 * p.K);
    a.th = tp.th;
    a.tw = tp.tw;
    a.tiles_y = tp.tiles_y;
    a.tiles_x = tp.tiles_x;
    a.lanes_shift = log2i(tp.lanes);
    a.R = tp.R;
    a.rh = tp.rh;
    a.rw = tp.rw;
    a.ps = tp.ps;
    a.nvp = tp.nvp;
    a.ps_magic = magic_for(tp.ps);
    a.npad_magic = magic_for(p.P - 3 * p.G * p.K);
    a.tw_magic = magic_for(tp.tw);
    for (int k = 0; k < p.K && k < kMaxTiledPoints; ++k) {
        const int kc = ((p.kw - 1) / 2) * p.kh + (p.kh - 1) / 2;   // centre of the full grid (i over kernel_w outer)
        const int kk = k + ((p.remove_center && k >= kc) ? 1 : 0);
        const int i = kk / p.kh, j = kk - i * p.kh;
        a.gdh[k] = (float)(j * p.dh);
        a.gdw[k] = (float)(i * p.dw);
    }
    a.ch = tp.ch;
    a.cw = tp.cw;
    a.ctiles_y = tp.ctiles_y;
    a.ctiles_x = tp.ctiles_x;
    a.cw_magic = magic_for(tp.cw);
    a.src_cap = tp.src_cap;
    a.gps = tp.gps;
    a.gps_magic = magic_for(tp.gps);
    a.rec_offset = tp.rec_offset;
    a.gs_offset = tp.gs_offset;
    return a;
}

// Shapes every tiled launch relies on (the planner only produces these).
bool out_tiles_ok(const Problem &p, const TilePlan &tp)
{
    return tp.threads % 64 == 0 && tp.threads <= kMaxTileThreads && tp.threads >= tp.th * tp.tw * tp.lanes &&
           tp.rw * tp.ps <= 64 * kMaxRowChunks && p.K <= 25 && tp.ps >= tp.nvp;
}

}  // namespace

hipError_t launch_forward_tiled(const Problem &p, const TilePlan &tp, const void *value, const void *offset_mask,
                                void *output, hipStream_t stream)
{
    if (!out_tiles_ok(p, tp))
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
        void (*k_)(TArgs) = p.K <= 9 ? (p.softmax ? dcnv4_fwd_tiled<T, D, 9, true> : dcnv4_fwd_tiled<T, D, 9, false>) \
                                     : (p.softmax ? dcnv4_fwd_tiled<T, D, 25, true> : dcnv4_fwd_tiled<T, D, 25, false>); \
        const hipError_t e_ =                                                                        \
            allow_dynamic_lds(reinterpret_cast<const void *>(k_), (size_t)tp.lds_bytes);             \
        if (e_ != hipSuccess)                                                                        \
            return e_;                                                                               \
        hipLaunchKernelGGL(k_, grid, block, tp.lds_bytes, stream, a);                                \
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

namespace {

typedef void (*Kernel)(TArgs);

template <typename T, int CG>
Kernel values_kernel(bool small_k, bool sm)
{
    if (small_k)
        return sm ? dcnv4_bwd_values_tiled<T, CG, 9, true> : dcnv4_bwd_values_tiled<T, CG, 9, false>;
    return sm ? dcnv4_bwd_values_tiled<T, CG, 25, true> : dcnv4_bwd_values_tiled<T, CG, 25, false>;
}

template <typename T>
Kernel values_kernel_for(int Cg, bool small_k, bool sm)
{
    switch (Cg) {
    case 4:
        if constexpr (sizeof(T) == 4)
            return values_kernel<T, 4>(small_k, sm);
        return nullptr;
    case 8:
        return values_kernel<T, 8>(small_k, sm);
    case 16:
        return values_kernel<T, 16>(small_k, sm);
    case 32:
        return values_kernel<T, 32>(small_k, sm);
    default:
        return nullptr;
    }
}

template <typename T, int DP>
Kernel offsets_kernel(bool small_k, bool sm)
{
    if (small_k)
        return sm ? dcnv4_bwd_offsets_tiled<T, DP, 9, true> : dcnv4_bwd_offsets_tiled<T, DP, 9, false>;
    return sm ? dcnv4_bwd_offsets_tiled<T, DP, 25, true> : dcnv4_bwd_offsets_tiled<T, DP, 25, false>;
}

template <typename T>
Kernel offsets_kernel_for(int dp, bool small_k, bool sm)
{
    switch (dp) {
    case 4:
        if constexpr (sizeof(T) == 4)
            return offsets_kernel<T, 4>(small_k, sm);
        return nullptr;
    case 8:
        return offsets_kernel<T, 8>(small_k, sm);
    case 16:
        return offsets_kernel<T, 16>(small_k, sm);
    default:
        return nullptr;
    }
}

}  // namespace

hipError_t launch_backward_tiled(const Problem &p, const TilePlan &tp, const void *value, const void *offset_mask,
                                 const void *grad_output, void *grad_value, void *grad_offset_mask,
                                 hipStream_t stream)
{
    const int es = p.elem;
    if (!out_tiles_ok(p, tp) || p.K > 25 || tp.tw * (p.P - 3 * p.G * p.K) > 64 * kMaxRowChunks ||
        tp.tw * 3 * p.K > 64 * kMaxRowChunks || tp.ch < 2 || tp.ch % 2 != 0 || tp.cw < 1 ||
        (tp.ch / 2) * tp.cw > kCellThreads || (tp.ch + 1) * (tp.cw + 1) >= kCellBinSlots || tp.src_cap < 1 ||
        tp.src_cap > kCellThreads || tp.gps * 16 < p.Cg * es ||
        tp.rec_offset < (kCellBinSlots + kCellThreads / 64) * 4 || tp.rec_offset % 16 != 0 ||
        tp.gs_offset < tp.rec_offset + tp.src_cap * p.K * 16 || tp.gs_offset % 16 != 0 ||
        tp.splat_lds_bytes < tp.gs_offset + tp.src_cap * tp.gps * 16 ||
        // source window width: within a batch and within a staged row
        (tp.cw + 2 * tp.R + (p.kw - 1) * p.dw + 1) / p.sw + 2 > tp.src_cap ||
        ((tp.cw + 2 * tp.R + (p.kw - 1) * p.dw + 1) / p.sw + 2) * tp.gps > 64 * kMaxRowChunks ||
        // the gradient rows of the tile (padded to whole 16-byte vectors per
        // pixel) reuse the value rows' LDS
        tp.th * tp.tw * ((3 * (p.K <= 9 ? 9 : 25) * es + 15) / 16 * 16) > tp.lds_bytes)
        return hipErrorInvalidConfiguration;
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
    const bool small_k = p.K <= 9, sm = p.softmax != 0;
    Kernel values = nullptr, offsets = nullptr;
    if (p.dtype == 0) {
        values = values_kernel_for<float>(p.Cg, small_k, sm);
        offsets = offsets_kernel_for<float>(tp.dp, small_k, sm);
    } else if (p.dtype == 1) {
        values = values_kernel_for<_Float16>(p.Cg, small_k, sm);
        offsets = offsets_kernel_for<_Float16>(tp.dp, small_k, sm);
    } else if (p.dtype == 2) {
        values = values_kernel_for<bf16_t>(p.Cg, small_k, sm);
        offsets = offsets_kernel_for<bf16_t>(tp.dp, small_k, sm);
    }
    if (!values || !offsets)
        return hipErrorInvalidValue;
    // 1) grad_value of near samples: every cell written once, plain stores
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
    // 2) grad_offset_mask, plus far samples' grad_value by device atomics
    {
        const int blocks = p.N * tp.tiles_y * tp.tiles_x * p.G;
        const hipError_t e = allow_dynamic_lds(reinterpret_cast<const void *>(offsets), (size_t)tp.lds_bytes);
        if (e != hipSuccess)
            return e;
        hipLaunchKernelGGL(offsets, dim3(blocks), dim3(tp.threads), tp.lds_bytes, stream, a);
    }
    return hipGetLastError();
}

}  // namespace dcnv4
