// Device-side helpers shared by the DCNv4 kernels (gfx950 / CDNA4).
#pragma once

#include <hip/hip_runtime.h>

// buffer_atomic_add_f32 through a buffer resource (the hardware range check
// drops lanes whose offset lies outside the resource).
__device__ float dcnv4_buffer_atomic_fadd(float v, __amdgpu_buffer_rsrc_t rsrc, int voffset, int soffset,
                                          int aux) __asm("llvm.amdgcn.raw.ptr.buffer.atomic.fadd.f32");


namespace dcnv4 {
namespace dev {

// dword3 of a raw (stride 0) buffer resource on gfx9-family devices.
constexpr int kRawBufferConfig = 0x00020000;

typedef unsigned int u32x4 __attribute__((ext_vector_type(4)));
typedef float f32x4 __attribute__((ext_vector_type(4)));
typedef unsigned int u32x2 __attribute__((ext_vector_type(2)));
typedef float f32x2 __attribute__((ext_vector_type(2)));
typedef _Float16 f16x8 __attribute__((ext_vector_type(8)));
// __builtin_bit_cast is only ever applied to whole vectors or scalars here;
// applied to a vector-element lvalue it reads element 0 with this compiler.

__device__ __forceinline__ __amdgpu_buffer_rsrc_t rsrc(const void *base, int bytes)
{
    return __builtin_amdgcn_make_buffer_rsrc(const_cast<void *>(base), 0, bytes, kRawBufferConfig);
}

__device__ __forceinline__ u32x4 load16(__amdgpu_buffer_rsrc_t r, unsigned off)
{
    return __builtin_amdgcn_raw_buffer_load_b128(r, off, 0, 0);
}

// Round-robin dispatch puts consecutive workgroups on different XCDs, each
// with its own L2.  Renumber so that XCD x processes one contiguous range of
// work items: neighbouring tiles sample overlapping value rows (and the
// groups of one tile share offset/mask lines), so their re-reads hit one L2.
__device__ __forceinline__ int xcd_tile(int b, int nb)
{
    const int xcd = b & 7, idx = b >> 3;
    const int per = nb >> 3, rem = nb & 7;
    return xcd * per + min(xcd, rem) + idx;
}

// ---- storage types -------------------------------------------------------

struct bf16_t {
    unsigned short bits;
};

__device__ __forceinline__ unsigned bf16_round(float f)
{
    // fp32 -> bf16 bits, round to nearest even (inputs are finite).
    const unsigned u = __builtin_bit_cast(unsigned, f);
    return (u + 0x7fffu + ((u >> 16) & 1u)) >> 16;
}

template <typename T>
struct Store;

template <>
struct Store<float> {
    __device__ static float scalar(float v) { return v; }
    __device__ static float make(float v) { return v; }
    __device__ static float get(const u32x4 *r, int c)
    {
        const f32x4 f = __builtin_bit_cast(f32x4, r[c >> 2]);
        return f[c & 3];
    }
    __device__ static void pack(const float *acc, u32x4 *r, int nv)
    {
        for (int v = 0; v < nv; ++v) {
            f32x4 f;
            for (int e = 0; e < 4; ++e)
                f[e] = acc[4 * v + e];
            r[v] = __builtin_bit_cast(u32x4, f);
        }
    }
};

template <>
struct Store<_Float16> {
    __device__ static float scalar(_Float16 v) { return (float)v; }
    __device__ static _Float16 make(float v) { return (_Float16)v; }   // round to nearest even
    __device__ static float from_bits(unsigned b) { return (float)__builtin_bit_cast(_Float16, (unsigned short)b); }
    __device__ static float get(const u32x4 *r, int c)
    {
        const f16x8 h = __builtin_bit_cast(f16x8, r[c >> 3]);
        return (float)h[c & 7];
    }
    __device__ static void pack(const float *acc, u32x4 *r, int nv)
    {
        for (int v = 0; v < nv; ++v) {
            f16x8 h;
            for (int e = 0; e < 8; ++e)
                h[e] = (_Float16)acc[8 * v + e];   // round to nearest even
            r[v] = __builtin_bit_cast(u32x4, h);
        }
    }
};

template <>
struct Store<bf16_t> {
    __device__ static float scalar(bf16_t v) { return __builtin_bit_cast(float, (unsigned)v.bits << 16); }
    __device__ static bf16_t make(float v) { return bf16_t{(unsigned short)bf16_round(v)}; }
    __device__ static float from_bits(unsigned b) { return __builtin_bit_cast(float, (b & 0xffffu) << 16); }
    __device__ static float get(const u32x4 *r, int c)
    {
        const unsigned w = r[c >> 3][(c & 7) >> 1];
        return __builtin_bit_cast(float, (c & 1) ? (w & 0xffff0000u) : (w << 16));
    }
    __device__ static void pack(const float *acc, u32x4 *r, int nv)
    {
        for (int v = 0; v < nv; ++v)
            for (int e = 0; e < 4; ++e)
                r[v][e] = bf16_round(acc[8 * v + 2 * e]) | (bf16_round(acc[8 * v + 2 * e + 1]) << 16);
    }
};

// ---- sampling geometry ----------------------------------------------------

// Scalars every kernel needs to place a sample.
struct Geom {
    int H, W, C, Ho, Wo;
    int kh, kw, sh, sw, ph, pw, dh, dw;
    int rc, kc;          // remove_center; index of the centre in the full grid
    float scale;         // offset_scale
};

// Grid indices (i over kernel_w, j over kernel_h) of the k-th sampling point.
__device__ __forceinline__ void grid_point(const Geom &g, int k, int &i, int &j)
{
    const int kk = k + ((g.rc && k >= g.kc) ? 1 : 0);
    i = kk / g.kh;
    j = kk - i * g.kh;
}

// Sample location: one fp32 fma per axis (the reference definition rounds
// the same way, so floor() agrees bit for bit).
struct Loc {
    float h, w;     // location
    int bh, bw;     // integer base: ho*sh - ph + j*dh, wo*sw - pw + i*dw
};

__device__ __forceinline__ Loc locate(const Geom &g, int ho, int wo, int k, float dx, float dy)
{
    int i, j;
    grid_point(g, k, i, j);
    Loc l;
    l.bh = ho * g.sh - g.ph + j * g.dh;
    l.bw = wo * g.sw - g.pw + i * g.dw;
    l.w = __builtin_fmaf(g.scale, dx, (float)l.bw);
    l.h = __builtin_fmaf(g.scale, dy, (float)l.bh);
    return l;
}

// A sample contributes only if loc lies in [-1,H) x [-1,W) (all four corners
// outside otherwise; NaN fails too).
__device__ __forceinline__ bool live(const Geom &g, const Loc &l)
{
    return l.h >= -1.0f && l.h < (float)g.H && l.w >= -1.0f && l.w < (float)g.W;
}

// Bilinear footprint of a live sample: the top-left corner, the fractional
// parts, and which of the two rows / two columns lie inside the image (a
// corner outside [0,H)x[0,W) has value 0: zero-extended image).
struct Footprint {
    int h0, w0;
    float lh, lw;            // loc - floor(loc)
    bool r0, r1, c0, c1;     // rows h0, h0+1 and columns w0, w0+1 inside the image
};

__device__ __forceinline__ Footprint footprint(const Geom &g, const Loc &l)
{
    Footprint f;
    const float fh = floorf(l.h), fw = floorf(l.w);
    f.h0 = (int)fh;
    f.w0 = (int)fw;
    f.lh = l.h - fh;
    f.lw = l.w - fw;
    f.r0 = f.h0 >= 0;
    f.r1 = f.h0 + 1 < g.H;
    f.c0 = f.w0 >= 0;
    f.c1 = f.w0 + 1 < g.W;
    return f;
}

// Byte offset of corner (h0, w0), channel offset included, inside a buffer
// holding images [0, N) of an (N,H,W,C) tensor.  Negative rows/columns of
// image 0 wrap to huge unsigned values and fail the buffer range check like
// offsets past the end; other out-of-image corners land on neighbouring
// pixels and must get a zero weight.
__device__ __forceinline__ unsigned corner_offset(const Geom &g, int n, const Footprint &f, int es, int chan_off)
{
    return ((unsigned)(n * g.H + f.h0) * (unsigned)g.W + (unsigned)f.w0) * (unsigned)(g.C * es) + (unsigned)chan_off;
}

// Corner weights m*w_q with corners outside the image set to 0 (values are
// finite by contract, so 0 * neighbouring data is 0).
__device__ __forceinline__ void masked_weights(const Footprint &f, float m, float &w00, float &w01, float &w10,
                                               float &w11)
{
    const float hh = f.r0 ? 1.0f - f.lh : 0.0f;
    const float lh = f.r1 ? f.lh : 0.0f;
    const float hw = f.c0 ? 1.0f - f.lw : 0.0f;
    const float lw = f.c1 ? f.lw : 0.0f;
    const float mh = m * hh, ml = m * lh;
    w00 = mh * hw;
    w01 = mh * lw;
    w10 = ml * hw;
    w11 = ml * lw;
}

}  // namespace dev
}  // namespace dcnv4
