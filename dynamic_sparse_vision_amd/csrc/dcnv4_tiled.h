// Shared pieces of the LDS-tiled DCNv4 kernels (gfx950 / CDNA4): kernel
// arguments, staging, offsets and masks in registers, sample placement,
// and the host-side argument packing.  The kernels live in
// dcnv4_tiled_fwd.hip, dcnv4_tiled_bwd_offsets.hip and
// dcnv4_tiled_bwd_values.hip; their launches in dcnv4_tiled_launch.hip.
//
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

#pragma once

#include "dcnv4_device.h"
#include "dcnv4_internal.h"

namespace dcnv4 {
namespace tiled {


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
    int gb, gb_shift;            // forward: groups per block (a power of two), log2
    int nvb, pst;                // forward: 16-byte vectors of a block's pixel slice; LDS pixel stride (slots)
    unsigned pst_magic;
    int R, rh, rw;               // halo radius; LDS value region, pixels
    int ps, nvp;                 // LDS pixel stride; data vectors per pixel (16-byte units)
    unsigned ps_magic;
    unsigned rw_magic;           // ceil(2^32 / rw)
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
    unsigned abias;   // LDS byte address of image pixel (0, 0) relative to the
                      // region, less 2^22 * (rowb + colb) (see biased_int)
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
    f.abias = 0u - (unsigned)(ry0 * f.rowb + rx0 * f.colb) - (1u << 22) * (unsigned)(f.rowb + f.colb);
    return f;
}

// An integer-valued float x with |x| < 2^22 as 2^22 + x in the low 24 bits
// (adding 1.5 * 2^23 puts x in the mantissa at unit scale): a float-to-int
// conversion that is defined for every input, at the cost of one add.
__device__ __forceinline__ unsigned biased_int(float x)
{
    return __builtin_bit_cast(unsigned, x + 12582912.0f);
}

// One sample in the main loops: location, floor, near test (false for NaN),
// and the LDS byte address of the top-left corner when near (of the grid
// position otherwise).
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
    // Floors are turned into integers by bit pattern (biased_int), which is
    // defined for any float: huge, infinite and NaN coordinates give some
    // address that the select then discards.  Near floors are below 2^22 in
    // magnitude (the tiled planner takes maps of at most 2^21 pixels a
    // side), so the biased addresses are exact modulo 2^32.
    const unsigned addr = __umul24(biased_int(s.fh), (unsigned)f.rowb) + __umul24(biased_int(s.fw), (unsigned)f.colb) +
                          f.abias;
    s.addr = s.nr ? (int)addr : 0;
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

inline unsigned magic_for(int d)
{
    // ceil(2^32 / d): mulhi(e, magic) == e / d for 0 <= e < 2^32 / d;
    // d == 1 is encoded as 0 (see divm)
    if (d <= 1)
        return 0u;
    return (unsigned)((((unsigned long long)1 << 32) + (unsigned)d - 1) / (unsigned)d);
}

inline int log2i(int v)
{
    int s = 0;
    while ((1 << s) < v)
        ++s;
    return s;
}

inline TArgs make_targs(const Problem &p, const TilePlan &tp)
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
    a.rw_magic = magic_for(tp.rw);
    a.gb = tp.gb > 0 ? tp.gb : 1;
    a.gb_shift = log2i(a.gb);
    a.nvb = a.gb * tp.nvp;
    a.pst = a.nvb | 1;
    a.pst_magic = magic_for(a.pst);
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
inline bool out_tiles_ok(const Problem &p, const TilePlan &tp)
{
    return tp.threads % 64 == 0 && tp.threads <= kMaxTileThreads && tp.threads >= tp.th * tp.tw * tp.lanes &&
           tp.rw * tp.ps <= 64 * kMaxRowChunks && p.K <= 25 && tp.ps >= tp.nvp;
}


typedef void (*Kernel)(TArgs);

// Instantiations, by storage dtype (enum dcnv4_dtype), channels per lane
// (dp) or per group (cg), K <= 9 (small_k) or K <= 25, and softmax mode;
// nullptr where none exists.
Kernel fwd_kernel(int dtype, int dp, bool small_k, bool sm);
Kernel bwd_offsets_kernel(int dtype, int dp, bool small_k, bool sm);
Kernel bwd_values_kernel(int dtype, int cg, bool small_k, bool sm);

}  // namespace tiled
}  // namespace dcnv4
