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
// of one image and gb consecutive groups (whose channels of a pixel make one
// 128-byte line where the channel count allows), stages those channels of
// the value rows under the tile's sampling grid plus a halo of R pixels into
// LDS once (zeros outside the image: the zero-extended image), and gathers
// corners from LDS.
//
// A sample whose 2x2 footprint lies in the staged region reads its corners
// there with no bounds test (corners outside the image read the staged
// zeros); any other live sample reads its corners from global memory after
// the main loop.  With R up to 5 and offsets of a few pixels these are a
// small share.  Each lane keeps its pixel's offsets and masks in registers,
// so the LDS holds value rows only.
//
// Staging uses direct-to-LDS buffer loads, one LDS row per group of wave
// instructions: slot j of every row comes from the row's base plus a
// per-lane offset that is the same for all rows, so a slot costs one add.
//
// Backward: device-scope fp32 atomics on this multi-XCD part are resolved
// beyond L2 and LDS fp32 atomics are slow, so grad_value of the samples
// within Rc of their grid position (|floor(loc) - grid position| <= Rc on
// both axes) is computed without float atomics: a block owns a tile of
// *input* cells, evaluates those samples of the output pixels that can
// reach it, sorts them by their top-left corner cell (a counting sort with
// integer LDS atomics), and every thread sums in registers, for a vertical
// pair of cells, the lists of the corner cells that reach them; the tile is
// then written with plain stores.  grad_offset_mask is forward-shaped; it
// also adds the grad_value contributions of the other live samples with
// device atomics (one wave instruction per sample), after the cell-tile
// kernel has written every cell.

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
    // output tiles
    int th, tw, tiles_y, tiles_x, lanes_shift;
    int gb, gb_shift;            // groups per block (a power of two), log2
    int nvb, pst;                // 16-byte vectors of a block's pixel slice; LDS pixel stride (slots)
    unsigned pst_magic;
    int R, rh, rw;               // halo radius of the LDS value region; its allocated size, pixels
    int Rc;                      // backward: near radius of the cell-tile kernel (see dcnv4_bwd_offsets_tiled)
    int cg_shift;                // log2(Cg) (the backward's Cg is a power of two)
    unsigned run_magic;          // ceil(2^32 / (gb * 3K)): a pixel's gradient run of a block
    unsigned half_magic;         // ceil(2^32 / (gb * 3K / 2))
    int nvp;                     // data vectors of a pixel and group (16-byte units)
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

// The LDS region of an output-tile block (forward, grad_offset_mask): the
// value rows and columns its samples can reach within a halo of R pixels of
// the tile's grid, clamped
// to the image plus a border of one pixel of zeros (rows -1 .. H, columns
// -1 .. W): corners beyond that border only belong to samples that are not
// live.  Region pixel (rr, cc) is image pixel (y0 + rr, x0 + cc).  A block
// covers gb consecutive groups, whose channels of a pixel are one contiguous
// slice of nvb 16-byte vectors (128 bytes, a whole cache line, where the
// channel count allows); the LDS holds the slice of region pixel (rr, cc)
// from 16-byte slot (rr * rw + cc) * pst, pst = nvb rounded up to odd (an
// odd pixel stride spreads random pixel reads over the LDS banks), rw being
// the region width the plan allocates (the widest region of any block).
struct Region {
    int y0, x0, rows, cols;
};

__device__ __forceinline__ Region tile_region(const TArgs &a, const Tile &t)
{
    const Geom &g = a.geo;
    const int y0u = t.oy0 * g.sh - g.ph - a.R, x0u = t.ox0 * g.sw - g.pw - a.R;
    const int hspan = (a.th - 1) * g.sh + (g.kh - 1) * g.dh + 2 * a.R + 2;
    const int wspan = (a.tw - 1) * g.sw + (g.kw - 1) * g.dw + 2 * a.R + 2;
    Region r;
    r.y0 = max(y0u, -1);
    r.x0 = max(x0u, -1);
    r.rows = min(y0u + hspan, g.H + 1) - r.y0;
    r.cols = min(x0u + wspan, g.W + 1) - r.x0;
    return r;
}

// Block -> (image, tile row, tile column, group block), group block
// fastest; t.g is the block's first group.
__device__ __forceinline__ Tile block_tile(const TArgs &a)
{
    int b = xcd_tile(blockIdx.x, gridDim.x);
    const int gblocks = a.G >> a.gb_shift;
    Tile t;
    t.g = (b % gblocks) << a.gb_shift;
    b /= gblocks;
    const int tx = b % a.tiles_x;
    b /= a.tiles_x;
    const int ty = b % a.tiles_y;
    t.n = b / a.tiles_y;
    t.oy0 = ty * a.th;
    t.ox0 = tx * a.tw;
    return t;
}

// Stage the block's slice of the region's pixels (zeros outside the image)
// with direct-to-LDS loads: consecutive lanes read consecutive 16-byte
// vectors of a pixel's slice, so a wave instruction covers whole cache lines.
// Waves take whole rows.
__device__ __forceinline__ void stage_region(const TArgs &a, const Tile &t, const Region &rg, char *lds, int es)
{
    const Geom &geo = a.geo;
    const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6, nwaves = blockDim.x >> 6;
    const int row_slots = rg.cols * a.pst;
    const unsigned cs = (unsigned)(geo.C * es), goff = (unsigned)(t.g * a.Cg * es);
    // slot j of a row: region column j / pst, vector j % pst (the last of an
    // even slice is the padding slot, zero)
    unsigned lo[kMaxRowChunks];
#pragma unroll
    for (int c = 0; c < kMaxRowChunks; ++c) {
        lo[c] = kOutOfRange;
        const int j = c * 64 + lane;
        if (j < row_slots) {
            const int cc = (int)divm((unsigned)j, a.pst_magic);
            const int v = j - cc * a.pst;
            const int x = rg.x0 + cc;
            if (v < a.nvb && (unsigned)x < (unsigned)geo.W)
                lo[c] = (unsigned)x * cs + goff + 16u * (unsigned)v;
        }
    }
    const __amdgpu_buffer_rsrc_t r = rsrc(a.value, a.value_bytes);
    const unsigned row_bytes = (unsigned)geo.W * cs;
    const int row_stride = a.rw * a.pst * 16;
    for (int rr = wave; rr < rg.rows; rr += nwaves) {
        const int y = rg.y0 + rr;
        const unsigned base = (unsigned)y < (unsigned)geo.H ? (unsigned)(t.n * geo.H + y) * row_bytes : kOutOfRange;
        char *dst = lds + rr * row_stride;
#pragma unroll
        for (int c = 0; c < kMaxRowChunks; ++c) {
            if (c * 64 < row_slots && c * 64 + lane < row_slots)
                dma<16>(r, dst + c * 64 * 16, (base == kOutOfRange || lo[c] == kOutOfRange) ? kOutOfRange : base + lo[c]);
        }
    }
}

// An integer-valued float x with |x| < 2^22 as 2^22 + x in the low 24 bits
// (adding 1.5 * 2^23 puts x in the mantissa at unit scale): a float-to-int
// conversion that is defined for every input, at the cost of one add.
__device__ __forceinline__ unsigned biased_int(float x)
{
    return __builtin_bit_cast(unsigned, x + 12582912.0f);
}

// A sample's location and its floor.
struct SampleLoc {
    float lh, lw, fh, fw;
};

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
    a.th = tp.th;
    a.tw = tp.tw;
    a.tiles_y = tp.tiles_y;
    a.tiles_x = tp.tiles_x;
    a.lanes_shift = log2i(tp.lanes);
    a.R = tp.R;
    a.rh = tp.rh;
    a.rw = tp.rw;
    a.nvp = tp.nvp;
    a.gb = tp.gb > 0 ? tp.gb : 1;
    a.gb_shift = log2i(a.gb);
    a.Rc = tp.Rc;
    a.cg_shift = log2i(p.Cg);
    a.run_magic = magic_for(a.gb * 3 * p.K);
    a.half_magic = magic_for(a.gb * 3 * p.K / 2);
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

typedef void (*Kernel)(TArgs);

// Instantiations, by storage dtype (enum dcnv4_dtype), channels per lane
// (dp) or per group (cg), K <= 9 (small_k) or K <= 25, and softmax mode;
// nullptr where none exists.
Kernel fwd_kernel(int dtype, int dp, bool small_k, bool sm);
Kernel bwd_offsets_kernel(int dtype, int dp, bool small_k, bool sm);
Kernel bwd_values_kernel(int dtype, int cg, bool small_k, bool sm);

}  // namespace tiled
}  // namespace dcnv4
