// HIP kernels of flash deformable attention (gfx950).
//
// Operation (multi-scale deformable attention, Zhu et al., "Deformable
// DETR", equation 3; named by the codewithpapers record of "Efficient
// Deformable ConvNets" through the official repository's
// flash_deform_attn_func.py): for each (image n, query q, head m) a softmax
// over the L*K attention logits weights L*K bilinear samples of head m's D
// channels, taken at column u*W_l - 1/2 and row v*H_l - 1/2 of level l.
//
// Layout and mapping:
//   * A "unit" is one (n, q, m); units are numbered head-major, (n, m, q),
//     so a block holds consecutive queries of one head, and the blocks of a
//     launch are renumbered XCD-aware, so each XCD works through a
//     contiguous range of (image, head) slices: the value rows one head of
//     one image can sample (S * D elements, 2.7 MB for four levels of an
//     800x1280 input at D = 32 fp32) stay in that XCD's L2.
//   * Forward: D/8 lanes per unit, 8 channels per lane (the D' channels per
//     thread and 128-bit loads of the walkthrough "DCNv4论文解析", section
//     2.2); a corner is one (fp16/bf16) or two (fp32) 128-bit buffer loads.
//     The softmax is taken once per unit, its lanes sharing the logits, into
//     LDS; with 16-bit storage the unit's lanes then place one sample each
//     and broadcast its corner offsets and weights to the others (fp32
//     lanes place every sample themselves, which measured faster there).
//   * Backward, with a caller workspace (the sorted path): the location and
//     logit gradients in the forward's mapping -- per sample, grad_output
//     dotted with each corner and summed over the unit's lanes by DPP, the
//     rest of the sample's arithmetic done by the lane that placed it --
//     which also emits each live sample's bin -- the cell of its top-left
//     corner -- and a 16-byte record; a counting sort per (image, head) slice, its
//     queries split over several blocks, each counting in LDS (the coarse
//     levels put hundreds of samples on one bin, which device atomics would
//     serialise) and merging into the slice's counts with one device atomic
//     per bin, then a scan and a placement pass; finally every value cell
//     sums the records of the four bins whose samples have it as a corner --
//     two runs of adjacent bins -- with D/4 lanes of four channels, and is
//     written once (a slice's coarsest level first: its cells have the
//     longest lists).
//   * Backward without a workspace (or when a slice's bins do not fit the
//     LDS): D lanes per unit, one channel each, and every (sample, corner,
//     channel) is a device fp32 atomic (N*Q*M*L*K*4*D of them, resolved
//     beyond the L2 on this part), coalesced over the D lanes.
//   * Every corner outside its level's map gets an out-of-range buffer
//     offset: its loads return 0 and its atomics are dropped by the buffer
//     range check, exactly the zero padding of the definition.
//   * Coordinates are one fp32 fma per axis (as in the definition used by
//     the tests); the softmax subtracts the maximum logit and uses expf.

#include "dcnv4_device.h"
#include "dcnv4_internal.h"
#include "fdattn_internal.h"

#include <algorithm>
#include <climits>
#include <type_traits>

namespace fdattn {
namespace {

using dcnv4::dev::bf16_t;
using dcnv4::dev::f32x2;
using dcnv4::dev::f32x4;
using dcnv4::dev::rsrc;
using dcnv4::dev::Store;
using dcnv4::dev::u32x2;
using dcnv4::dev::u32x4;
using dcnv4::dev::xcd_tile;

constexpr unsigned kOutOfRange = 0x80000000u;   // beyond any launch's buffer
constexpr int kSortThreads = 1024;               // one block per (image, head) slice
constexpr size_t kSortLdsMax = 150 * 1024;       // bin counters of one slice, LDS bytes
constexpr int kSortUnroll = 4;                   // samples per thread and round of the count and place loops
// rounds of the scan (four bins per thread each) that cover the most bins
// the LDS sort admits
constexpr int kScanRounds = (int)((kSortLdsMax / sizeof(unsigned) + 4 * kSortThreads - 1) / (4 * kSortThreads));
#ifndef FDATTN_GATHER_CHANNELS
#define FDATTN_GATHER_CHANNELS 4
#endif
constexpr int kGatherChannels = FDATTN_GATHER_CHANNELS;   // channels per lane in the grad_value gather (2 or 4)

struct Args {
    const void *value;
    const void *loc_attn;
    const void *grad_out;
    void *out;
    float *grad_value;
    void *grad_loc;
    int units;            // N*Q*M
    int Q, M, D, K, L, LK, P;
    unsigned value_bytes; // bytes of value in this launch
    unsigned gv_bytes;    // bytes of grad_value in this launch
    unsigned img_bytes;   // bytes of one image of value
    unsigned gv_img_bytes;
    unsigned pix_bytes;   // bytes of one value pixel (all heads)
    int elem_bytes;       // bytes of the storage type
    int S;
    int lvl_h[kMaxLevels], lvl_w[kMaxLevels], lvl_start[kMaxLevels];
    // sorted grad_value path: bins of top-left corner cells, (H_l + 1) x
    // (W_l + 1) per level (rows and columns -1 .. size-1), nbs per slice
    int nbs;
    int lvl_bin[kMaxLevels];
    unsigned *counts;     // [N*M*nbs]: counts, then bin ends
    unsigned *starts;     // [N*M*nbs]: first record of each bin
    unsigned *bases;      // [N*M*sb*nbs]: a sort block's offset inside each bin
    unsigned *keys;       // [N*M*Q*L*K]: each sample's bin (or ~0u), in (n, m, q, i) order
    f32x4 *urecs;         // [N*M*Q*L*K]: each sample's record, same order
    f32x4 *recs;          // [N*M*Q*L*K]: (a*(1-ly), a*ly, lx, query), sorted by bin
    int sb;               // sort blocks per slice
};

template <typename T>
__device__ __forceinline__ float ld1(const T *p)
{
    return Store<T>::scalar(*p);
}

// Two consecutive entries (a location pair; the row base is 16-byte aligned
// and the pair starts at an even entry).
__device__ __forceinline__ void ld2(const float *p, float &a, float &b)
{
    const f32x2 v = *reinterpret_cast<const f32x2 *>(p);
    a = v[0];
    b = v[1];
}
__device__ __forceinline__ void ld2(const _Float16 *p, float &a, float &b)
{
    const unsigned w = *reinterpret_cast<const unsigned *>(p);
    a = Store<_Float16>::from_bits(w & 0xffffu);
    b = Store<_Float16>::from_bits(w >> 16);
}
__device__ __forceinline__ void ld2(const bf16_t *p, float &a, float &b)
{
    const unsigned w = *reinterpret_cast<const unsigned *>(p);
    a = Store<bf16_t>::from_bits(w & 0xffffu);
    b = Store<bf16_t>::from_bits(w >> 16);
}

// CPL (2 or 4) consecutive channels as floats; the address is aligned to
// CPL elements.
template <typename T, int CPL>
__device__ __forceinline__ void load_channels(const T *p, float *out)
{
    if constexpr (CPL == 2) {
        ld2(p, out[0], out[1]);
    } else if constexpr (sizeof(T) == 4) {
        const f32x4 v = *reinterpret_cast<const f32x4 *>(p);
        for (int c = 0; c < 4; ++c)
            out[c] = v[c];
    } else {
        const u32x2 v = *reinterpret_cast<const u32x2 *>(p);
        for (int c = 0; c < 4; ++c)
            out[c] = Store<T>::from_bits((v[c >> 1] >> (16 * (c & 1))) & 0xffffu);
    }
}

__device__ __forceinline__ void st2(float *p, float a, float b)
{
    f32x2 v;
    v[0] = a;
    v[1] = b;
    *reinterpret_cast<f32x2 *>(p) = v;
}
__device__ __forceinline__ void st2(_Float16 *p, float a, float b)
{
    const unsigned lo = __builtin_bit_cast(unsigned short, (_Float16)a);
    const unsigned hi = __builtin_bit_cast(unsigned short, (_Float16)b);
    *reinterpret_cast<unsigned *>(p) = lo | (hi << 16);
}
__device__ __forceinline__ void st2(bf16_t *p, float a, float b)
{
    *reinterpret_cast<unsigned *>(p) = dcnv4::dev::bf16_round(a) | (dcnv4::dev::bf16_round(b) << 16);
}

// Softmax statistics of a unit's logits: maximum and 1 / sum exp(z - max).
template <typename T>
__device__ __forceinline__ void softmax_stats(const T *logits, int n, float &mx, float &inv)
{
    mx = -__builtin_huge_valf();
    for (int i = 0; i < n; ++i)
        mx = fmaxf(mx, ld1(logits + i));
    float sum = 0.0f;
    for (int i = 0; i < n; ++i)
        sum += expf(ld1(logits + i) - mx);
    inv = 1.0f / sum;
}

// Bilinear footprint of one sample: corner byte offsets (relative to the
// corner (r0, c0) = offset `o00`; out-of-map corners -> kOutOfRange) and the
// fp32 weights hy*hx, hy*lx, ly*hx, ly*lx.
struct Corners {
    unsigned o[4];
    float w[4];
    float ly, lx, hy, hx;
    int r0, c0;
};

__device__ __forceinline__ Corners corners(float y, float x, int H, int W, int start, unsigned pix_bytes,
                                           unsigned base)
{
    Corners c;
    const float fy = floorf(y), fx = floorf(x);
    const int r0 = (int)fy, c0 = (int)fx;
    c.r0 = r0;
    c.c0 = c0;
    c.ly = y - fy;
    c.lx = x - fx;
    c.hy = 1.0f - c.ly;
    c.hx = 1.0f - c.lx;
    c.w[0] = c.hy * c.hx;
    c.w[1] = c.hy * c.lx;
    c.w[2] = c.ly * c.hx;
    c.w[3] = c.ly * c.lx;
    const bool rv0 = r0 >= 0, rv1 = r0 + 1 < H, cv0 = c0 >= 0, cv1 = c0 + 1 < W;
    // valid corners lie inside the launch's buffer; the unsigned wrap of an
    // invalid corner's offset is never used
    const unsigned o00 = base + (unsigned)(start + r0 * W + c0) * pix_bytes;
    const unsigned orow = (unsigned)W * pix_bytes;
    c.o[0] = (rv0 && cv0) ? o00 : kOutOfRange;
    c.o[1] = (rv0 && cv1) ? o00 + pix_bytes : kOutOfRange;
    c.o[2] = (rv1 && cv0) ? o00 + orow : kOutOfRange;
    c.o[3] = (rv1 && cv1) ? o00 + orow + pix_bytes : kOutOfRange;
    return c;
}

__device__ __forceinline__ bool live(float y, float x, float Hf, float Wf)
{
    return y >= -1.0f && y < Hf && x >= -1.0f && x < Wf;   // false for NaN
}

// Eight channels of a corner as floats.
template <typename T>
__device__ __forceinline__ void load8(__amdgpu_buffer_rsrc_t r, unsigned off, float *v);

template <>
__device__ __forceinline__ void load8<float>(__amdgpu_buffer_rsrc_t r, unsigned off, float *v)
{
    const f32x4 a = __builtin_bit_cast(f32x4, dcnv4::dev::load16(r, off));
    const f32x4 b = __builtin_bit_cast(f32x4, dcnv4::dev::load16(r, off + 16u));
    for (int e = 0; e < 4; ++e) {
        v[e] = a[e];
        v[4 + e] = b[e];
    }
}

template <typename T>
__device__ __forceinline__ void load8_16(__amdgpu_buffer_rsrc_t r, unsigned off, float *v)
{
    const u32x4 q = dcnv4::dev::load16(r, off);
    for (int e = 0; e < 4; ++e) {
        v[2 * e] = Store<T>::from_bits(q[e] & 0xffffu);
        v[2 * e + 1] = Store<T>::from_bits(q[e] >> 16);
    }
}

template <>
__device__ __forceinline__ void load8<_Float16>(__amdgpu_buffer_rsrc_t r, unsigned off, float *v)
{
    load8_16<_Float16>(r, off, v);
}

template <>
__device__ __forceinline__ void load8<bf16_t>(__amdgpu_buffer_rsrc_t r, unsigned off, float *v)
{
    load8_16<bf16_t>(r, off, v);
}

// One channel of a corner as a float (backward).
template <typename T>
__device__ __forceinline__ float load1(__amdgpu_buffer_rsrc_t r, unsigned off)
{
    if constexpr (sizeof(T) == 4)
        return __builtin_bit_cast(float, __builtin_amdgcn_raw_buffer_load_b32(r, off, 0, 0));
    else
        return Store<T>::from_bits(__builtin_amdgcn_raw_buffer_load_b16(r, off, 0, 0));
}

// Sum over the `lanes` lanes of a unit (aligned groups, a power of two).
__device__ __forceinline__ float unit_sum(float x, int lanes)
{
    if (lanes >= 2)
        x += __builtin_bit_cast(float, __builtin_amdgcn_mov_dpp(__builtin_bit_cast(int, x), 0xB1, 0xF, 0xF, false));
    if (lanes >= 4)
        x += __builtin_bit_cast(float, __builtin_amdgcn_mov_dpp(__builtin_bit_cast(int, x), 0x4E, 0xF, 0xF, false));
    for (int d = 4; d < lanes; d <<= 1)
        x += __shfl_xor(x, d);
    return x;
}

// Maximum over the `lanes` lanes of a unit (aligned groups, a power of two).
__device__ __forceinline__ float unit_max(float x, int lanes)
{
    if (lanes >= 2)
        x = fmaxf(x, __builtin_bit_cast(float, __builtin_amdgcn_mov_dpp(__builtin_bit_cast(int, x), 0xB1, 0xF, 0xF, false)));
    if (lanes >= 4)
        x = fmaxf(x, __builtin_bit_cast(float, __builtin_amdgcn_mov_dpp(__builtin_bit_cast(int, x), 0x4E, 0xF, 0xF, false)));
    for (int d = 4; d < lanes; d <<= 1)
        x = fmaxf(x, __shfl_xor(x, d));
    return x;
}

// The attention weights of a unit: a softmax over its n logits, each of the
// unit's `lanes` lanes taking every lanes-th one, written to att_s; a weight
// is exp(z - mx) * inv.  The unit's lanes are one wave: its LDS accesses are
// performed in order, and the fences only keep the compiler's order, so
// every lane may read any weight afterwards.
template <typename T>
__device__ __forceinline__ void unit_softmax(const T *logits, int n, int lane, int lanes, float *att_s, float &mx,
                                             float &inv)
{
    mx = -__builtin_huge_valf();
    for (int j = lane; j < n; j += lanes)
        mx = fmaxf(mx, ld1(logits + j));
    mx = unit_max(mx, lanes);
    float sum = 0.0f;
    for (int j = lane; j < n; j += lanes) {
        const float e = expf(ld1(logits + j) - mx);
        att_s[j] = e;
        sum += e;
    }
    inv = 1.0f / unit_sum(sum, lanes);
    for (int j = lane; j < n; j += lanes)
        att_s[j] *= inv;
    __builtin_amdgcn_fence(__ATOMIC_RELEASE, "wavefront");
    __builtin_amdgcn_wave_barrier();
    __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "wavefront");
}

// Lane R's value of x in every lane of its aligned group of U lanes.  Groups
// of two and four lanes use a DPP quad permutation, wider ones a
// permute through the LDS crossbar.
template <int U, int R>
__device__ __forceinline__ unsigned group_bcast(unsigned x)
{
    if constexpr (U == 1) {
        return x;
    } else if constexpr (U == 2) {
        return (unsigned)__builtin_amdgcn_mov_dpp((int)x, R | R << 2 | (2 + R) << 4 | (2 + R) << 6, 0xF, 0xF, false);
    } else if constexpr (U == 4) {
        return (unsigned)__builtin_amdgcn_mov_dpp((int)x, R * 0x55, 0xF, 0xF, false);
    } else {
        const int src = (int)(__lane_id() & ~(unsigned)(U - 1)) | R;
        return (unsigned)__builtin_amdgcn_ds_bpermute(src << 2, (int)x);
    }
}

// f(integral_constant<int, 0>) .. f(integral_constant<int, N - 1>), in order.
template <int N, int I = 0, typename F>
__device__ __forceinline__ void static_for(F &&f)
{
    if constexpr (I < N) {
        f(std::integral_constant<int, I>{});
        static_for<N, I + 1>(f);
    }
}

// ---- forward --------------------------------------------------------------

template <typename T, int U>
__global__ __launch_bounds__(kThreads) void fdattn_fwd(Args a)
{
    extern __shared__ float att_lds[];   // [units per block][LK]: attention weights
    constexpr int es = (int)sizeof(T);
    constexpr int upb = kThreads / U;
    const int blk = xcd_tile(blockIdx.x, gridDim.x);
    const int unit = blk * upb + (int)threadIdx.x / U;
    const int lane = (int)threadIdx.x % U;
    if (unit >= a.units)
        return;
    const int nm = unit / a.Q;
    const int n = nm / a.M;
    const int m = nm - n * a.M;
    const size_t qrow = ((size_t)n * a.Q + (unit - nm * a.Q)) * a.M + m;   // (n, q, m) row
    const int LK = a.LK;
    const T *row = static_cast<const T *>(a.loc_attn) + qrow * a.P;
    float *att_s = att_lds + ((int)threadIdx.x / U) * LK;
    float mx, inv;
    unit_softmax(row + 2 * LK, LK, lane, U, att_s, mx, inv);

    const __amdgpu_buffer_rsrc_t vr = rsrc(a.value, (int)a.value_bytes);
    // corner offsets are the unit's (its image and head); each lane adds its
    // channels' offset to them
    const unsigned base = (unsigned)n * a.img_bytes + (unsigned)(m * a.D * es);
    const unsigned chan = (unsigned)(lane * 8 * es);
    float acc[8];
    for (int c = 0; c < 8; ++c)
        acc[c] = 0.0f;
    if constexpr (es == 4) {
        // fp32: every lane of the unit places every sample itself (two
        // 128-bit loads per corner; measured faster for fp32 than the
        // broadcast below, 344 against 354 us on the 800x1280 workload)
        for (int l = 0; l < a.L; ++l) {
            const int H = a.lvl_h[l], W = a.lvl_w[l], start = a.lvl_start[l];
            const float Hf = (float)H, Wf = (float)W;
            const int i0 = l * a.K;
#pragma unroll 4
            for (int k = 0; k < a.K; ++k) {
                const int i = i0 + k;
                float u, v;
                ld2(row + 2 * i, u, v);
                const float x = __builtin_fmaf(u, Wf, -0.5f);
                const float y = __builtin_fmaf(v, Hf, -0.5f);
                const bool in = live(y, x, Hf, Wf);
                const float att = att_s[i];
                // a dead sample (huge or NaN location included) is placed at
                // (-1, -1): only bounded floors are converted to integers
                const Corners c = corners(in ? y : -1.0f, in ? x : -1.0f, H, W, start, a.pix_bytes, base);
                float vq[4][8];
#pragma unroll
                for (int qq = 0; qq < 4; ++qq)   // kOutOfRange plus a channel offset stays out of range
                    load8<T>(vr, (in ? c.o[qq] : kOutOfRange) + chan, vq[qq]);
                const float a0 = in ? att * c.w[0] : 0.0f, a1 = in ? att * c.w[1] : 0.0f;
                const float a2 = in ? att * c.w[2] : 0.0f, a3 = in ? att * c.w[3] : 0.0f;
                for (int e = 0; e < 8; ++e) {
                    float s = acc[e];
                    s = __builtin_fmaf(a0, vq[0][e], s);
                    s = __builtin_fmaf(a1, vq[1][e], s);
                    s = __builtin_fmaf(a2, vq[2][e], s);
                    acc[e] = __builtin_fmaf(a3, vq[3][e], s);
                }
            }
        }
    } else {
        // The U lanes of a unit take U samples at a time: each lane places one
        // (location, bilinear weights times the attention weight, corner
        // offsets), then the group reads the four corners of each of the U
        // samples in turn, its offsets and weights broadcast from the lane that
        // placed it.  No branch: a sample outside its map, or past the level's
        // last point, gets zero weights and out-of-range offsets (whose loads
        // return zeros), so the compiler can overlap the loads of the samples.
        for (int l = 0; l < a.L; ++l) {
            const int H = a.lvl_h[l], W = a.lvl_w[l], start = a.lvl_start[l];
            const float Hf = (float)H, Wf = (float)W;
            const int i0 = l * a.K;
            for (int kb = 0; kb < a.K; kb += U) {
                const bool have = kb + lane < a.K;
                const int i = i0 + (have ? kb + lane : a.K - 1);
                float u, v;
                ld2(row + 2 * i, u, v);
                const float x = __builtin_fmaf(u, Wf, -0.5f);
                const float y = __builtin_fmaf(v, Hf, -0.5f);
                const bool in = have && live(y, x, Hf, Wf);
                const float att = att_s[i];
                // a dead sample (huge or NaN location included) is placed at
                // (-1, -1): only bounded floors are converted to integers
                const Corners c = corners(in ? y : -1.0f, in ? x : -1.0f, H, W, start, a.pix_bytes, base);
                unsigned o[4], w[4];
#pragma unroll
                for (int q = 0; q < 4; ++q) {
                    o[q] = in ? c.o[q] : kOutOfRange;
                    w[q] = __builtin_bit_cast(unsigned, in ? att * c.w[q] : 0.0f);
                }
                static_for<U>([&](auto r) {
                    constexpr int R = decltype(r)::value;
                    float vq[4][8], wq[4];
#pragma unroll
                    for (int q = 0; q < 4; ++q) {
                        // kOutOfRange plus a channel offset stays out of range
                        load8<T>(vr, group_bcast<U, R>(o[q]) + chan, vq[q]);
                        wq[q] = __builtin_bit_cast(float, group_bcast<U, R>(w[q]));
                    }
                    for (int e = 0; e < 8; ++e) {
                        float s = acc[e];
                        s = __builtin_fmaf(wq[0], vq[0][e], s);
                        s = __builtin_fmaf(wq[1], vq[1][e], s);
                        s = __builtin_fmaf(wq[2], vq[2][e], s);
                        acc[e] = __builtin_fmaf(wq[3], vq[3][e], s);
                    }
                });
            }
        }
    }
    T *out = static_cast<T *>(a.out) + qrow * a.D + lane * 8;
    u32x4 r[2];
    Store<T>::pack(acc, r, 8 * es / 16);
    reinterpret_cast<u32x4 *>(out)[0] = r[0];
    if (es == 4)
        reinterpret_cast<u32x4 *>(out)[1] = r[1];
}

// ---- backward -------------------------------------------------------------

template <typename T>
__global__ __launch_bounds__(kThreads) void fdattn_bwd(Args a)
{
    extern __shared__ float ga_lds[];   // [units per block][LK]: sum_d grad_out_d * sample_d
    constexpr int es = (int)sizeof(T);
    const int D = a.D;
    const int upb = kThreads / D;
    const int blk = xcd_tile(blockIdx.x, gridDim.x);
    const int lu = (int)threadIdx.x / D;
    const int lane = (int)threadIdx.x - lu * D;
    const int unit = blk * upb + lu;
    if (unit >= a.units)
        return;   // whole units leave together; lane sums stay inside a unit
    const int nm = unit / a.Q;
    const int n = nm / a.M;
    const int m = nm - n * a.M;
    const size_t qrow = ((size_t)n * a.Q + (unit - nm * a.Q)) * a.M + m;   // (n, q, m) row
    const int LK = a.LK;
    const T *row = static_cast<const T *>(a.loc_attn) + qrow * a.P;
    T *grow = static_cast<T *>(a.grad_loc) + qrow * a.P;
    float *ga = ga_lds + lu * LK;
    float mx, inv;
    softmax_stats(row + 2 * LK, LK, mx, inv);
    const float g = ld1(static_cast<const T *>(a.grad_out) + qrow * D + lane);

    const __amdgpu_buffer_rsrc_t vr = rsrc(a.value, (int)a.value_bytes);
    const __amdgpu_buffer_rsrc_t gr = rsrc(a.grad_value, (int)a.gv_bytes);
    const unsigned vbase = (unsigned)n * a.img_bytes + (unsigned)((m * D + lane) * es);
    const unsigned gbase = (unsigned)n * a.gv_img_bytes + (unsigned)((m * D + lane) * 4);
    float dot = 0.0f;
    int i = 0;
    for (int l = 0; l < a.L; ++l) {
        const int H = a.lvl_h[l], W = a.lvl_w[l], start = a.lvl_start[l];
        const float Hf = (float)H, Wf = (float)W;
        for (int k = 0; k < a.K; ++k, ++i) {
            float u, v;
            ld2(row + 2 * i, u, v);
            const float x = __builtin_fmaf(u, Wf, -0.5f);
            const float y = __builtin_fmaf(v, Hf, -0.5f);
            const float att = expf(ld1(row + 2 * LK + i) - mx) * inv;
            float gs = 0.0f, gx = 0.0f, gy = 0.0f;
            if (live(y, x, Hf, Wf)) {   // the same for every lane of the unit
                const Corners c = corners(y, x, H, W, start, a.pix_bytes, vbase);
                const float v0 = load1<T>(vr, c.o[0]);
                const float v1 = load1<T>(vr, c.o[1]);
                const float v2 = load1<T>(vr, c.o[2]);
                const float v3 = load1<T>(vr, c.o[3]);
                const float s = c.w[0] * v0 + c.w[1] * v1 + c.w[2] * v2 + c.w[3] * v3;
                const float dxv = c.hy * (v1 - v0) + c.ly * (v3 - v2);
                const float dyv = c.hx * (v2 - v0) + c.lx * (v3 - v1);
                gs = g * s;
                gx = g * dxv;
                gy = g * dyv;
                // grad_value: the same corner offsets in the fp32 tensor
                const float ag = att * g;
                for (int q = 0; q < 4; ++q) {
                    const unsigned go = c.o[q] == kOutOfRange
                                            ? kOutOfRange
                                            : (c.o[q] - vbase) / es * 4 + gbase;
                    dcnv4_buffer_atomic_fadd(ag * c.w[q], gr, (int)go, 0, 0);
                }
            }
            gs = unit_sum(gs, D);
            gx = unit_sum(gx, D);
            gy = unit_sum(gy, D);
            dot += att * gs;
            if (lane == (i & (D - 1))) {
                st2(grow + 2 * i, att * Wf * gx, att * Hf * gy);
                ga[i] = gs;
            }
        }
    }
    // logits: a_i (g_i - sum_j a_j g_j); lane i % D wrote ga[i] itself
    for (int j = lane; j < LK; j += D) {
        const float att = expf(ld1(row + 2 * LK + j) - mx) * inv;
        grow[2 * LK + j] = Store<T>::make(att * (ga[j] - dot));
    }
    for (int e = 3 * LK + lane; e < a.P; e += D)
        grow[e] = Store<T>::make(0.0f);
}

// Location and logit gradients, plus each sample's bin and record for the
// grad_value sort: the forward's mapping, U = D/8 lanes of 8 channels per
// unit, 128-bit corner loads, lane sums of eight lanes or fewer by DPP, and
// a branch-free sample loop (dead samples: out-of-range loads, results
// selected to 0).  With ST the block's bins and records are staged in LDS
// and written out as one contiguous range at the end (the units of a block
// are consecutive); otherwise each goes straight to memory.
template <typename T, int U, bool ST>
__global__ __launch_bounds__(kThreads) void fdattn_bwd_loc(Args a)
{
    extern __shared__ f32x4 lds4[];
    constexpr int es = (int)sizeof(T);
    constexpr int upb = kThreads / U;
    const int LK = a.LK;
    char *lds = reinterpret_cast<char *>(lds4);
    f32x4 *rec_lds = lds4;                                                            // [upb * LK] (ST)
    unsigned *key_lds = reinterpret_cast<unsigned *>(lds + (ST ? upb * LK * 16 : 0));  // [upb * LK] (ST)
    float *ga_lds = reinterpret_cast<float *>(lds + (ST ? upb * LK * 20 : 0));        // [upb * LK]
    T *grow_lds = reinterpret_cast<T *>(lds + upb * LK * (ST ? 24 : 4));              // [upb * P] (ST)
    const int blk = xcd_tile(blockIdx.x, gridDim.x);
    const int lu = (int)threadIdx.x / U;
    const int lane = (int)threadIdx.x % U;
    const int unit = blk * upb + lu;
    // whole units are valid or not; lane sums stay inside a unit
    if (unit < a.units) {
    const int nm = unit / a.Q;
    const int n = nm / a.M;
    const int m = nm - n * a.M;
    const size_t qrow = ((size_t)n * a.Q + (unit - nm * a.Q)) * a.M + m;   // (n, q, m) row
    const T *row = static_cast<const T *>(a.loc_attn) + qrow * a.P;
    T *grow = ST ? grow_lds + lu * a.P : static_cast<T *>(a.grad_loc) + qrow * a.P;
    float *ga = ga_lds + lu * LK;
    // the attention weights, in the slots of the lane sums: sample i's
    // weight is read by every lane of the unit before one lane overwrites it
    // with the sample's sum (in program order, and the lanes are one wave)
    float mx, inv;
    unit_softmax(row + 2 * LK, LK, lane, U, ga, mx, inv);
    float g[8];
    {
        const u32x4 *gp = reinterpret_cast<const u32x4 *>(static_cast<const T *>(a.grad_out) + qrow * a.D + lane * 8);
        const u32x4 g0 = gp[0];
        const u32x4 g1 = es == 4 ? gp[1] : u32x4{0u, 0u, 0u, 0u};
        const u32x4 gv[2] = {g0, g1};
        for (int e = 0; e < 8; ++e)
            g[e] = Store<T>::get(gv, e);
    }
    const __amdgpu_buffer_rsrc_t vr = rsrc(a.value, (int)a.value_bytes);
    const unsigned base = (unsigned)n * a.img_bytes + (unsigned)((m * a.D + lane * 8) * es);
    float dot = 0.0f;
    for (int l = 0; l < a.L; ++l) {
        const int H = a.lvl_h[l], W = a.lvl_w[l], start = a.lvl_start[l];
        const float Hf = (float)H, Wf = (float)W;
        const int i0 = l * a.K;
        for (int k = 0; k < a.K; ++k) {
            const int i = i0 + k;
            float u, v;
            ld2(row + 2 * i, u, v);
            const float x = __builtin_fmaf(u, Wf, -0.5f);
            const float y = __builtin_fmaf(v, Hf, -0.5f);
            const bool in = live(y, x, Hf, Wf);
            const float att = ga[i];
            // a dead sample (huge or NaN location included) is placed at
            // (-1, -1): only bounded floors are converted to integers
            const Corners c = corners(in ? y : -1.0f, in ? x : -1.0f, H, W, start, a.pix_bytes, base);
            float v0[8], v1[8], v2[8], v3[8];
            load8<T>(vr, in ? c.o[0] : kOutOfRange, v0);
            load8<T>(vr, in ? c.o[1] : kOutOfRange, v1);
            load8<T>(vr, in ? c.o[2] : kOutOfRange, v2);
            load8<T>(vr, in ? c.o[3] : kOutOfRange, v3);
            // grad_output dotted with each corner's channels, summed over
            // the unit's lanes; the sample's value and its derivatives along
            // x and y are linear in the corners, so their products with
            // grad_output follow from these four sums
            float t0 = 0.0f, t1 = 0.0f, t2 = 0.0f, t3 = 0.0f;
            for (int e = 0; e < 8; ++e) {
                t0 = __builtin_fmaf(g[e], v0[e], t0);
                t1 = __builtin_fmaf(g[e], v1[e], t1);
                t2 = __builtin_fmaf(g[e], v2[e], t2);
                t3 = __builtin_fmaf(g[e], v3[e], t3);
            }
            t0 = unit_sum(t0, U);
            t1 = unit_sum(t1, U);
            t2 = unit_sum(t2, U);
            t3 = unit_sum(t3, U);
            const float gs = in ? c.w[0] * t0 + c.w[1] * t1 + c.w[2] * t2 + c.w[3] * t3 : 0.0f;
            const float gx = in ? c.hy * (t1 - t0) + c.ly * (t3 - t2) : 0.0f;
            const float gy = in ? c.hx * (t2 - t0) + c.lx * (t3 - t1) : 0.0f;
            dot += att * gs;
            if (lane == (i & (U - 1))) {
                st2(grow + 2 * i, att * Wf * gx, att * Hf * gy);
                ga[i] = gs;
                // the sample's bin and record for the grad_value sort
                const unsigned key = in ? (unsigned)(a.lvl_bin[l] + (c.r0 + 1) * (W + 1) + (c.c0 + 1)) : ~0u;
                f32x4 rec;
                rec[0] = att * c.hy;
                rec[1] = att * c.ly;
                rec[2] = c.lx;
                rec[3] = __builtin_bit_cast(float, (unsigned)(unit - nm * a.Q));
                if (ST) {
                    key_lds[lu * LK + i] = key;
                    rec_lds[lu * LK + i] = rec;
                } else {
                    const size_t si = (size_t)unit * LK + i;
                    a.keys[si] = key;
                    a.urecs[si] = rec;
                }
            }
        }
    }
    // logits: a_i (g_i - sum_j a_j g_j); lane i % U wrote ga[i] itself
    for (int j = lane; j < LK; j += U) {
        const float att = expf(ld1(row + 2 * LK + j) - mx) * inv;
        grow[2 * LK + j] = Store<T>::make(att * (ga[j] - dot));
    }
    for (int e = 3 * LK + lane; e < a.P; e += U)
        grow[e] = Store<T>::make(0.0f);
    }
    if (ST) {
        __syncthreads();
        const int u0 = blk * upb;
        const int nu = min(upb, a.units - u0);
        const int nv = nu * LK;
        const size_t si0 = (size_t)u0 * LK;
        for (int t = (int)threadIdx.x; t < nv; t += kThreads) {
            a.keys[si0 + t] = key_lds[t];
            a.urecs[si0 + t] = rec_lds[t];
        }
        // the units' gradient rows, whole 16-byte vectors (rows are
        // contiguous, one per unit, at (n, q, m))
        const int rv = a.P * es / 16;
        const u32x4 *src = reinterpret_cast<const u32x4 *>(grow_lds);
        for (int t = (int)threadIdx.x; t < nu * rv; t += kThreads) {
            const int u = t / rv, v = t - u * rv;
            const int un = u0 + u;
            const int unm = un / a.Q;
            const int un_n = unm / a.M;
            const size_t r = ((size_t)un_n * a.Q + (un - unm * a.Q)) * a.M + (unm - un_n * a.M);
            reinterpret_cast<u32x4 *>(static_cast<T *>(a.grad_loc) + r * a.P)[v] = src[u * rv + v];
        }
    }
}

// Inclusive prefix sum over the 64 lanes of a wave (DPP row shifts, then
// row broadcasts; lanes without a source add 0).
__device__ __forceinline__ unsigned wave_prefix(unsigned v)
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

// The sort of the sorted grad_value path: a slice's queries are split over
// `sb` blocks; bins are the top-left corner cells, nbs per slice.
//   fdattn_count: each block counts its samples per bin in LDS, then adds
//     every non-zero count to the slice's global count with one device
//     atomic, whose returned value is the block's offset inside the bin.
//   fdattn_scan:  one block per slice turns the global counts into bin
//     starts (offset by the slice's first record slot, slice * Q * L * K)
//     and ends.
//   fdattn_place: each block starts its LDS cursors at bin start + its
//     offset and writes one record per sample.
// The coarse levels put hundreds of samples on one bin; the LDS atomics take
// those, and the device atomics see at most sb per bin.

// Samples [s0, s1) of block `sbi` of a slice, as indices into keys / urecs.
__device__ __forceinline__ void sort_range(const Args &a, int slice, int sbi, size_t &s0, size_t &s1)
{
    const size_t n = (size_t)a.Q * a.LK, per = (n + a.sb - 1) / a.sb;
    const size_t first = (size_t)slice * n;
    s0 = first + std::min(n, sbi * per);
    s1 = first + std::min(n, sbi * per + per);
}

__global__ __launch_bounds__(kSortThreads) void fdattn_count(Args a)
{
    extern __shared__ unsigned bins[];   // [nbs]
    const int slice = blockIdx.x / a.sb, sbi = blockIdx.x - slice * a.sb;
    const int tid = (int)threadIdx.x;
    for (int i = tid; i < a.nbs; i += kSortThreads)
        bins[i] = 0u;
    __syncthreads();
    size_t s0, s1;
    sort_range(a, slice, sbi, s0, s1);
    // kSortUnroll keys per thread are loaded before their counts are added,
    // so the loads' latency is paid once per kSortUnroll rounds
    for (size_t si0 = s0 + tid; si0 < s1; si0 += kSortUnroll * kSortThreads) {
        unsigned b[kSortUnroll];
#pragma unroll
        for (int u = 0; u < kSortUnroll; ++u) {
            const size_t si = si0 + (size_t)u * kSortThreads;
            b[u] = si < s1 ? a.keys[si] : ~0u;
        }
#pragma unroll
        for (int u = 0; u < kSortUnroll; ++u)
            if (b[u] != ~0u)
                __hip_atomic_fetch_add(bins + b[u], 1u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_WORKGROUP);
    }
    __syncthreads();
    unsigned *gcount = a.counts + (size_t)slice * a.nbs;
    unsigned *base = a.bases + ((size_t)slice * a.sb + sbi) * a.nbs;
    for (int i = tid; i < a.nbs; i += kSortThreads) {
        const unsigned c = bins[i];
        if (c)
            base[i] = __hip_atomic_fetch_add(gcount + i, c, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
    }
}

__global__ __launch_bounds__(kSortThreads) void fdattn_scan(Args a)
{
    __shared__ unsigned wsum[kSortThreads / 64];
    const int slice = blockIdx.x;
    const int tid = (int)threadIdx.x, lane = tid & 63, wave = tid >> 6;
    unsigned *cnt = a.counts + (size_t)slice * a.nbs;   // counts in, bin ends out
    unsigned *st = a.starts + (size_t)slice * a.nbs;
    // every count of the slice is loaded first (four per thread and round;
    // the slice's bins fit the LDS, so at most kScanRounds rounds), then the
    // rounds are scanned one after the other
    unsigned c[kScanRounds][4];
#pragma unroll
    for (int r = 0; r < kScanRounds; ++r)
#pragma unroll
        for (int e = 0; e < 4; ++e) {
            const int i = r * 4 * kSortThreads + 4 * tid + e;
            c[r][e] = i < a.nbs ? cnt[i] : 0u;
        }
    unsigned carry = (unsigned)slice * (unsigned)(a.Q * a.LK);
#pragma unroll
    for (int r = 0; r < kScanRounds; ++r) {
        if (r * 4 * kSortThreads >= a.nbs)
            break;
        const int i0 = r * 4 * kSortThreads + 4 * tid;
        const unsigned mine = c[r][0] + c[r][1] + c[r][2] + c[r][3];
        const unsigned x = wave_prefix(mine);
        if (lane == 63)
            wsum[wave] = x;
        __syncthreads();
        unsigned off = carry, tot = 0;
        for (int w = 0; w < kSortThreads / 64; ++w) {
            off += w < wave ? wsum[w] : 0u;
            tot += wsum[w];
        }
        unsigned e0 = off + x - mine;
#pragma unroll
        for (int e = 0; e < 4; ++e) {
            if (i0 + e < a.nbs) {
                st[i0 + e] = e0;
                cnt[i0 + e] = e0 + c[r][e];
            }
            e0 += c[r][e];
        }
        carry += tot;
        __syncthreads();   // wsum is rewritten by the next round
    }
}

__global__ __launch_bounds__(kSortThreads) void fdattn_place(Args a)
{
    extern __shared__ unsigned cursor[];   // [nbs]
    const int slice = blockIdx.x / a.sb, sbi = blockIdx.x - slice * a.sb;
    const int tid = (int)threadIdx.x;
    // bins this block has no sample in get a meaningless cursor (their
    // offset entry was never written) and are never used
    const unsigned *st = a.starts + (size_t)slice * a.nbs;
    const unsigned *base = a.bases + ((size_t)slice * a.sb + sbi) * a.nbs;
    for (int i = tid; i < a.nbs; i += kSortThreads)
        cursor[i] = st[i] + base[i];
    __syncthreads();
    size_t s0, s1;
    sort_range(a, slice, sbi, s0, s1);
    // kSortUnroll samples per thread: keys and records are loaded before
    // their places are taken
    for (size_t si0 = s0 + tid; si0 < s1; si0 += kSortUnroll * kSortThreads) {
        unsigned b[kSortUnroll];
        f32x4 r[kSortUnroll];
#pragma unroll
        for (int u = 0; u < kSortUnroll; ++u) {
            const size_t si = si0 + (size_t)u * kSortThreads;
            b[u] = ~0u;
            r[u] = f32x4{0.0f, 0.0f, 0.0f, 0.0f};
            if (si < s1) {
                b[u] = a.keys[si];
                r[u] = a.urecs[si];
            }
        }
#pragma unroll
        for (int u = 0; u < kSortUnroll; ++u) {
            if (b[u] != ~0u) {
                const unsigned idx =
                    __hip_atomic_fetch_add(cursor + b[u], 1u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_WORKGROUP);
                a.recs[idx] = r[u];
            }
        }
    }
}

// D/CPL lanes per value cell (CPL channels each, so a wave holds several
// cells and as many independent load chains): the cell is the top-left,
// top-right, bottom-left and bottom-right corner of the samples in bins
// (r, c), (r, c-1), (r-1, c) and (r-1, c-1); bins (r, c-1), (r, c) and
// (r-1, c-1), (r-1, c) are adjacent, so the cell reads two runs, taken as
// one list D/CPL records at a time, one per lane (coalesced), each reduced
// to (its weight for this cell, its query) and staged in LDS, from where the
// unit's lanes read them back as broadcasts.  Every cell is written once (no
// fill).
template <typename T, int CPL>
__global__ __launch_bounds__(kThreads) void fdattn_gather(Args a)
{
    extern __shared__ f32x2 stage_lds[];   // [units per block][D/CPL]: (weight, query)
    const int D = a.D;
    const int UL = D / CPL;   // lanes per cell
    const int upb = kThreads / UL;
    const int blk = xcd_tile(blockIdx.x, gridDim.x);
    const int lu = (int)threadIdx.x / UL;
    const int lane = (int)threadIdx.x - lu * UL;
    const int unit = blk * upb + lu;
    const int cells = a.units / a.Q * a.S;   // N*M*S
    if (unit >= cells)
        return;
    f32x2 *stage = stage_lds + lu * UL;
    const int slice = unit / a.S;
    const int n = slice / a.M;
    const int m = slice - n * a.M;
    // the cells of a slice are taken from the coarsest level to the finest:
    // the coarse cells' long lists start early instead of ending the launch
    int rc = unit - slice * a.S;
    int l = a.L - 1;
    while (l > 0 && rc >= a.lvl_h[l] * a.lvl_w[l]) {
        rc -= a.lvl_h[l] * a.lvl_w[l];
        --l;
    }
    const int W = a.lvl_w[l];
    const int s = a.lvl_start[l] + rc;
    const int r = rc / W, c = rc - r * W;
    const size_t bin_lc = (size_t)slice * a.nbs + a.lvl_bin[l] + (size_t)(r + 1) * (W + 1) + c;   // bin (r, c-1)
    const size_t bin_ulc = bin_lc - (W + 1);                                                         // bin (r-1, c-1)
    const T *gq = static_cast<const T *>(a.grad_out) + (size_t)n * a.Q * a.M * D + m * D + CPL * lane;
    const size_t qstride = (size_t)a.M * D;
    float acc[CPL];
#pragma unroll
    for (int c = 0; c < CPL; ++c)
        acc[c] = 0.0f;
    // The two runs -- bins (r, c-1), (r, c): the cell is in the records'
    // upper row; bins (r-1, c-1), (r-1, c): in their lower row -- are read
    // as one list, D/CPL records at a time: record j of the list is the j-th of
    // run 1, then of run 2.  In each run the records of the first bin have
    // this cell as their right column (weight lx), the others as their left
    // (1 - lx).  The grad_out loads of a batch go out eight at a time.
    const unsigned s1 = a.starts[bin_lc], m1 = a.counts[bin_lc], e1 = a.counts[bin_lc + 1];
    const unsigned s2 = a.starts[bin_ulc], m2 = a.counts[bin_ulc], e2 = a.counts[bin_ulc + 1];
    const unsigned n1 = e1 - s1, ntot = n1 + (e2 - s2);
    for (unsigned base = 0; base < ntot; base += (unsigned)UL) {
        const unsigned j = base + (unsigned)lane;
        f32x2 mine = {0.0f, 0.0f};
        if (j < ntot) {
            const bool run1 = j < n1;
            const unsigned idx = run1 ? s1 + j : s2 + (j - n1);
            const f32x4 rec = a.recs[idx];
            const float wy = run1 ? rec[0] : rec[1];
            mine[0] = wy * (idx < (run1 ? m1 : m2) ? rec[2] : 1.0f - rec[2]);
            mine[1] = rec[3];   // the query, as bits
        }
        // the unit's lanes are one wave: LDS accesses of a wave are
        // performed in order, the barriers only keep the compiler's order
        __builtin_amdgcn_wave_barrier();
        stage[lane] = mine;
        __builtin_amdgcn_fence(__ATOMIC_RELEASE, "wavefront");
        __builtin_amdgcn_wave_barrier();
        __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "wavefront");
        const int cnt = (int)min((unsigned)UL, ntot - base);
        for (int t0 = 0; t0 < cnt; t0 += 8) {
            float g[8][CPL], w[8];
#pragma unroll
            for (int u = 0; u < 8; ++u) {
                const int t = min(t0 + u, cnt - 1);   // repeats the last record: a valid row
                const f32x2 wq = stage[t];
                w[u] = t0 + u < cnt ? wq[0] : 0.0f;
                load_channels<T, CPL>(gq + __builtin_bit_cast(u32x2, wq)[1] * qstride, g[u]);   // whole-vector cast, then index
            }
#pragma unroll
            for (int u = 0; u < 8; ++u)
#pragma unroll
                for (int c = 0; c < CPL; ++c)
                    acc[c] = t0 + u < cnt ? __builtin_fmaf(w[u], g[u][c], acc[c]) : acc[c];
        }
        __builtin_amdgcn_wave_barrier();
    }
    float *gvp = a.grad_value + ((size_t)n * a.S + s) * qstride + m * D + CPL * lane;
    if constexpr (CPL == 4) {
        f32x4 out;
        for (int c = 0; c < 4; ++c)
            out[c] = acc[c];
        *reinterpret_cast<f32x4 *>(gvp) = out;
    } else {
        f32x2 out;
        out[0] = acc[0];
        out[1] = acc[1];
        *reinterpret_cast<f32x2 *>(gvp) = out;
    }
}

Args make_args(const Problem &p)
{
    Args a;
    a.units = p.N * p.Q * p.M;
    a.Q = p.Q;
    a.M = p.M;
    a.D = p.D;
    a.K = p.K;
    a.L = p.L;
    a.LK = p.L * p.K;
    a.P = p.P;
    a.pix_bytes = (unsigned)(p.M * p.D * p.elem);
    a.elem_bytes = p.elem;
    a.img_bytes = (unsigned)p.S * a.pix_bytes;
    a.gv_img_bytes = (unsigned)p.S * (unsigned)(p.M * p.D * 4);
    a.value_bytes = a.img_bytes * (unsigned)p.N;
    a.gv_bytes = a.gv_img_bytes * (unsigned)p.N;
    a.S = p.S;
    a.nbs = 0;
    for (int l = 0; l < kMaxLevels; ++l) {
        a.lvl_h[l] = l < p.L ? p.lvl_h[l] : 0;
        a.lvl_w[l] = l < p.L ? p.lvl_w[l] : 0;
        a.lvl_start[l] = l < p.L ? p.lvl_start[l] : 0;
        a.lvl_bin[l] = a.nbs;
        if (l < p.L)
            a.nbs += (p.lvl_h[l] + 1) * (p.lvl_w[l] + 1);
    }
    a.counts = nullptr;
    a.starts = nullptr;
    a.bases = nullptr;
    a.keys = nullptr;
    a.urecs = nullptr;
    a.recs = nullptr;
    // enough sort blocks to give every CU one (one block per CU fits the
    // bin counters), at most 16 per slice
    const int slices = p.N * p.M;
    a.sb = std::max(1, std::min(16, std::min(p.Q, (256 + slices - 1) / std::max(1, slices))));
    return a;
}

template <typename T>
hipError_t launch_fwd_t(const Args &a, hipStream_t stream)
{
    const int U = a.D / 8;
    const int upb = kThreads / U;
    const int blocks = (a.units + upb - 1) / upb;
    const size_t lds = (size_t)upb * a.LK * sizeof(float);   // attention weights
    void (*fn)(Args) = nullptr;
    switch (U) {
    case 1: fn = fdattn_fwd<T, 1>; break;
    case 2: fn = fdattn_fwd<T, 2>; break;
    case 4: fn = fdattn_fwd<T, 4>; break;
    case 8: fn = fdattn_fwd<T, 8>; break;
    case 16: fn = fdattn_fwd<T, 16>; break;
    default: return hipErrorInvalidValue;
    }
    const hipError_t e = dcnv4::allow_dynamic_lds(reinterpret_cast<const void *>(fn), lds);
    if (e != hipSuccess)
        return e;
    hipLaunchKernelGGL(fn, dim3(blocks), dim3(kThreads), lds, stream, a);
    return hipGetLastError();
}

template <typename T, bool ST>
hipError_t launch_bwd_loc_st(const Args &a, int blocks, size_t lds, hipStream_t stream)
{
    void (*fn)(Args) = nullptr;
    switch (a.D / 8) {
    case 1: fn = fdattn_bwd_loc<T, 1, ST>; break;
    case 2: fn = fdattn_bwd_loc<T, 2, ST>; break;
    case 4: fn = fdattn_bwd_loc<T, 4, ST>; break;
    case 8: fn = fdattn_bwd_loc<T, 8, ST>; break;
    default: return hipErrorInvalidValue;
    }
    const hipError_t e = dcnv4::allow_dynamic_lds(reinterpret_cast<const void *>(fn), lds);
    if (e != hipSuccess)
        return e;
    hipLaunchKernelGGL(fn, dim3(blocks), dim3(kThreads), lds, stream, a);
    return hipGetLastError();
}

template <typename T>
hipError_t launch_bwd_loc_t(const Args &a, hipStream_t stream)
{
    const int upb = kThreads / (a.D / 8);
    const int blocks = (a.units + upb - 1) / upb;
    const size_t ga = (size_t)upb * a.LK * sizeof(float);   // attention weights, then lane sums
    const size_t staged = ga + (size_t)upb * a.LK * (sizeof(unsigned) + sizeof(f32x4)) +
                          (size_t)upb * a.P * (a.elem_bytes);
    if (staged <= 64 * 1024)
        return launch_bwd_loc_st<T, true>(a, blocks, staged, stream);
    return launch_bwd_loc_st<T, false>(a, blocks, ga, stream);
}

// The sorted grad_value path applies when a slice's bin counters fit the LDS.
bool sort_fits(const Args &a)
{
    return (size_t)a.nbs * sizeof(unsigned) <= kSortLdsMax;
}

template <typename T>
hipError_t launch_bwd_t(const Args &a, hipStream_t stream)
{
    const int upb = kThreads / a.D;
    const int blocks = (a.units + upb - 1) / upb;
    const size_t lds = (size_t)upb * a.LK * sizeof(float);
    if (!a.recs) {
        hipLaunchKernelGGL((fdattn_bwd<T>), dim3(blocks), dim3(kThreads), lds, stream, a);
        return hipGetLastError();
    }
    hipError_t e = launch_bwd_loc_t<T>(a, stream);
    if (e != hipSuccess)
        return e;
    const int slices = a.units / a.Q;
    const size_t sort_lds = (size_t)a.nbs * sizeof(unsigned);
    e = dcnv4::allow_dynamic_lds(reinterpret_cast<const void *>(&fdattn_count), sort_lds);
    if (e == hipSuccess)
        e = dcnv4::allow_dynamic_lds(reinterpret_cast<const void *>(&fdattn_place), sort_lds);
    if (e != hipSuccess)
        return e;
    hipLaunchKernelGGL(fdattn_count, dim3(slices * a.sb), dim3(kSortThreads), sort_lds, stream, a);
    e = hipGetLastError();
    if (e != hipSuccess)
        return e;
    hipLaunchKernelGGL(fdattn_scan, dim3(slices), dim3(kSortThreads), 0, stream, a);
    e = hipGetLastError();
    if (e != hipSuccess)
        return e;
    hipLaunchKernelGGL(fdattn_place, dim3(slices * a.sb), dim3(kSortThreads), sort_lds, stream, a);
    e = hipGetLastError();
    if (e != hipSuccess)
        return e;
    const int cells = slices * a.S;
    const int gupb = kThreads / (a.D / kGatherChannels);
    hipLaunchKernelGGL((fdattn_gather<T, kGatherChannels>), dim3((cells + gupb - 1) / gupb), dim3(kThreads),
                       (size_t)kThreads * sizeof(f32x2), stream, a);
    return hipGetLastError();
}

}  // namespace

hipError_t launch_forward(const Problem &p, const void *value, const void *loc_attn, void *output,
                          hipStream_t stream)
{
    Args a = make_args(p);
    a.value = value;
    a.loc_attn = loc_attn;
    a.out = output;
    switch (p.dtype) {
    case 0: return launch_fwd_t<float>(a, stream);
    case 1: return launch_fwd_t<_Float16>(a, stream);
    case 2: return launch_fwd_t<bf16_t>(a, stream);
    default: return hipErrorInvalidValue;
    }
}

size_t workspace_bytes(const Problem &p)
{
    const Args a = make_args(p);
    if (!sort_fits(a))
        return 0;   // the atomic path: no workspace
    // counts/ends, starts, per-block offsets, records; whole 256-byte blocks
    const size_t nb = ((size_t)p.N * p.M * a.nbs + 63) / 64 * 64;
    const size_t nbb = ((size_t)p.N * p.M * a.sb * a.nbs + 63) / 64 * 64;
    const size_t ns = ((size_t)p.N * p.M * p.Q * p.L * p.K + 63) / 64 * 64;   // samples
    return (2 * nb + nbb + ns) * sizeof(unsigned) + 2 * ns * sizeof(f32x4);
}

hipError_t launch_backward(const Problem &p, const void *value, const void *loc_attn, const void *grad_output,
                           float *grad_value, void *grad_loc_attn, void *workspace, hipStream_t stream)
{
    Args a = make_args(p);
    a.value = value;
    a.loc_attn = loc_attn;
    a.grad_out = grad_output;
    a.grad_value = grad_value;
    a.grad_loc = grad_loc_attn;
    if (workspace && sort_fits(a)) {
        const size_t nb = ((size_t)p.N * p.M * a.nbs + 63) / 64 * 64;
        const size_t nbb = ((size_t)p.N * p.M * a.sb * a.nbs + 63) / 64 * 64;
        const size_t ns = ((size_t)p.N * p.M * p.Q * p.L * p.K + 63) / 64 * 64;
        a.counts = static_cast<unsigned *>(workspace);
        a.starts = a.counts + nb;
        a.bases = a.starts + nb;
        a.keys = a.bases + nbb;
        a.urecs = reinterpret_cast<f32x4 *>(a.keys + ns);
        a.recs = a.urecs + ns;
        // the global counts start at zero (the per-block offsets and bin
        // starts are written before they are read)
        const hipError_t e = dcnv4::launch_zero(a.counts, nb * sizeof(unsigned), stream);
        if (e != hipSuccess)
            return e;
    } else {
        const hipError_t e = dcnv4::launch_zero(grad_value, (size_t)a.gv_bytes, stream);
        if (e != hipSuccess)
            return e;
    }
    switch (p.dtype) {
    case 0: return launch_bwd_t<float>(a, stream);
    case 1: return launch_bwd_t<_Float16>(a, stream);
    case 2: return launch_bwd_t<bf16_t>(a, stream);
    default: return hipErrorInvalidValue;
    }
}

}  // namespace fdattn
