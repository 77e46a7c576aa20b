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
//   * Backward: D lanes per unit, one channel per lane, so the grad_value
//     atomics of one corner cover D contiguous floats (coalesced device
//     atomics); the location and logit gradients are lane sums (DPP).
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

namespace fdattn {
namespace {

using dcnv4::dev::bf16_t;
using dcnv4::dev::f32x2;
using dcnv4::dev::f32x4;
using dcnv4::dev::rsrc;
using dcnv4::dev::Store;
using dcnv4::dev::u32x4;
using dcnv4::dev::xcd_tile;

constexpr unsigned kOutOfRange = 0x80000000u;   // beyond any launch's buffer

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
    int lvl_h[kMaxLevels], lvl_w[kMaxLevels], lvl_start[kMaxLevels];
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
};

__device__ __forceinline__ Corners corners(float y, float x, int H, int W, int start, unsigned pix_bytes,
                                           unsigned base)
{
    Corners c;
    const float fy = floorf(y), fx = floorf(x);
    const int r0 = (int)fy, c0 = (int)fx;
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

// ---- forward --------------------------------------------------------------

template <typename T, int U>
__global__ __launch_bounds__(kThreads) void fdattn_fwd(Args a)
{
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
    float mx, inv;
    softmax_stats(row + 2 * LK, LK, mx, inv);

    const __amdgpu_buffer_rsrc_t vr = rsrc(a.value, (int)a.value_bytes);
    const unsigned base = (unsigned)n * a.img_bytes + (unsigned)((m * a.D + lane * 8) * es);
    float acc[8];
    for (int c = 0; c < 8; ++c)
        acc[c] = 0.0f;
    // The sample loop has no branch: a sample outside its map gets zero
    // weights and out-of-range offsets, so the compiler can overlap the
    // loads of several samples.
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
            const float att = expf(ld1(row + 2 * LK + i) - mx) * inv;
            Corners c = corners(y, x, H, W, start, a.pix_bytes, base);
            float v0[8], v1[8], v2[8], v3[8];
            load8<T>(vr, in ? c.o[0] : kOutOfRange, v0);
            load8<T>(vr, in ? c.o[1] : kOutOfRange, v1);
            load8<T>(vr, in ? c.o[2] : kOutOfRange, v2);
            load8<T>(vr, in ? c.o[3] : kOutOfRange, v3);
            const float a0 = in ? att * c.w[0] : 0.0f, a1 = in ? att * c.w[1] : 0.0f;
            const float a2 = in ? att * c.w[2] : 0.0f, a3 = in ? att * c.w[3] : 0.0f;
            for (int e = 0; e < 8; ++e) {
                float s = acc[e];
                s = __builtin_fmaf(a0, v0[e], s);
                s = __builtin_fmaf(a1, v1[e], s);
                s = __builtin_fmaf(a2, v2[e], s);
                acc[e] = __builtin_fmaf(a3, v3[e], s);
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
                    if (c.w[q] != 0.0f)
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
    a.img_bytes = (unsigned)p.S * a.pix_bytes;
    a.gv_img_bytes = (unsigned)p.S * (unsigned)(p.M * p.D * 4);
    a.value_bytes = a.img_bytes * (unsigned)p.N;
    a.gv_bytes = a.gv_img_bytes * (unsigned)p.N;
    for (int l = 0; l < kMaxLevels; ++l) {
        a.lvl_h[l] = l < p.L ? p.lvl_h[l] : 0;
        a.lvl_w[l] = l < p.L ? p.lvl_w[l] : 0;
        a.lvl_start[l] = l < p.L ? p.lvl_start[l] : 0;
    }
    return a;
}

template <typename T>
hipError_t launch_fwd_t(const Args &a, hipStream_t stream)
{
    const int U = a.D / 8;
    const int upb = kThreads / U;
    const int blocks = (a.units + upb - 1) / upb;
    switch (U) {
    case 1: hipLaunchKernelGGL((fdattn_fwd<T, 1>), dim3(blocks), dim3(kThreads), 0, stream, a); break;
    case 2: hipLaunchKernelGGL((fdattn_fwd<T, 2>), dim3(blocks), dim3(kThreads), 0, stream, a); break;
    case 4: hipLaunchKernelGGL((fdattn_fwd<T, 4>), dim3(blocks), dim3(kThreads), 0, stream, a); break;
    case 8: hipLaunchKernelGGL((fdattn_fwd<T, 8>), dim3(blocks), dim3(kThreads), 0, stream, a); break;
    case 16: hipLaunchKernelGGL((fdattn_fwd<T, 16>), dim3(blocks), dim3(kThreads), 0, stream, a); break;
    default: return hipErrorInvalidValue;
    }
    return hipGetLastError();
}

template <typename T>
hipError_t launch_bwd_t(const Args &a, hipStream_t stream)
{
    const int upb = kThreads / a.D;
    const int blocks = (a.units + upb - 1) / upb;
    const size_t lds = (size_t)upb * a.LK * sizeof(float);
    hipLaunchKernelGGL((fdattn_bwd<T>), dim3(blocks), dim3(kThreads), lds, stream, a);
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

hipError_t launch_backward(const Problem &p, const void *value, const void *loc_attn, const void *grad_output,
                           float *grad_value, void *grad_loc_attn, hipStream_t stream)
{
    Args a = make_args(p);
    a.value = value;
    a.loc_attn = loc_attn;
    a.grad_out = grad_output;
    a.grad_value = grad_value;
    a.grad_loc = grad_loc_attn;
    hipError_t e = dcnv4::launch_zero(grad_value, (size_t)a.gv_bytes, stream);
    if (e != hipSuccess)
        return e;
    switch (p.dtype) {
    case 0: return launch_bwd_t<float>(a, stream);
    case 1: return launch_bwd_t<_Float16>(a, stream);
    case 2: return launch_bwd_t<bf16_t>(a, stream);
    default: return hipErrorInvalidValue;
    }
}

}  // namespace fdattn
