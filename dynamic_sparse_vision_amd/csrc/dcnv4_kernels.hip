// HIP kernels of the DCNv4 spatial aggregation for gfx950 (CDNA4).
//
// Operation ("Efficient Deformable ConvNets", DCNv3 recap equation of the
// CSDN walkthrough "DCNv4论文解析", section 1.2, without the softmax of
// section 2.1): for each output pixel, group g and grid point k, a bilinear
// sample of the channel-last value tensor at
//   (ho*stride_h - pad_h + j*dil_h + s*dy,  wo*stride_w - pad_w + i*dil_w + s*dx)
// with zero padding, times an unnormalised scalar m, summed over k.
//
// Mapping (the method's own memory-access ideas, walkthrough section 2.2 and
// the blog "DCNv4架构解析", section "并行计算架构设计", kept where they hold on
// CDNA4):
//   * one thread owns DP contiguous channels of one (pixel, group): offsets,
//     masks and bilinear coefficients are read/computed once per DP channels;
//   * corner rows are fetched with 128-bit buffer loads (channel-last layout
//     makes the DP channels of a corner contiguous);
//   * the offset/mask rows of a block's pixels are staged in LDS with
//     coalesced 128-bit loads (rows are 16-byte multiples by the pad-to-8
//     rule), and read from LDS per grid point;
//   * fp32 coordinates (one fma, bit-identical to the reference definition),
//     fp32 weights and fp32 accumulation; RNE rounding on the store.
// CDNA4-specific choices: raw buffer resources give a hardware range check,
// so corners outside the tensor read 0 (and atomics outside it are dropped)
// without branches; the workgroup -> tile map is XCD-aware; no MFMA (a
// gather-weighted sum is not a dense contraction).

#include "dcnv4_internal.h"

#include <hip/hip_runtime.h>

// buffer_atomic_add_f32 through a buffer resource (the hardware range check
// drops lanes whose offset lies outside the resource).
__device__ float buffer_atomic_fadd(float v, __amdgpu_buffer_rsrc_t rsrc, int voffset, int soffset,
                                    int aux) __asm("llvm.amdgcn.raw.ptr.buffer.atomic.fadd.f32");

namespace dcnv4 {
namespace {

// dword3 of a raw (stride 0) buffer resource on gfx9-family devices.
constexpr int kRawBufferConfig = 0x00020000;

typedef unsigned int u32x4 __attribute__((ext_vector_type(4)));
typedef float f32x4 __attribute__((ext_vector_type(4)));
typedef _Float16 f16x8 __attribute__((ext_vector_type(8)));
// Note: __builtin_bit_cast is only ever applied to whole vectors or scalars
// here; applied to a vector-element lvalue it reads element 0 with this
// compiler.


struct KArgs {
    const void *value;
    const void *om;
    void *out;            // forward output
    const float *gout;    // backward: grad_output
    float *gvalue;        // backward: grad_value
    float *gom;           // backward: grad_offset_mask
    int H, W, Ho, Wo, G, Cg, C, K, P;
    int kh, sh, sw, ph, pw, dh, dw;
    int rc, kc;           // remove_center, index of the centre in the full grid
    float scale;
    int lanes, pix_per_block, total_pix;
    int value_bytes;      // bytes of value (and of grad_value) in this launch
};

// Round-robin dispatch puts consecutive workgroups on different XCDs, each
// with its own L2.  Renumber so that XCD x processes one contiguous range of
// tiles: neighbouring pixel tiles sample overlapping value rows, and those
// re-reads then hit the same L2.
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

template <typename T>
struct Store;

template <>
struct Store<float> {
    __device__ static float scalar(float v) { return v; }
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

__device__ __forceinline__ unsigned bf16_round(float f)
{
    // fp32 -> bf16 bits, round to nearest even (inputs are finite).
    const unsigned u = __builtin_bit_cast(unsigned, f);
    return (u + 0x7fffu + ((u >> 16) & 1u)) >> 16;
}

template <>
struct Store<bf16_t> {
    __device__ static float scalar(bf16_t v) { return __builtin_bit_cast(float, (unsigned)v.bits << 16); }
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

// Copy rows [pix0, pix0+npix) of the offset_mask tensor into LDS.
template <typename T>
__device__ __forceinline__ void stage_rows(const KArgs &a, int pix0, int npix, u32x4 *dst)
{
    const u32x4 *src = reinterpret_cast<const u32x4 *>(static_cast<const T *>(a.om) + (size_t)pix0 * a.P);
    const int nvec = npix * a.P * (int)sizeof(T) / 16;
    for (int i = threadIdx.x; i < nvec; i += blockDim.x)
        dst[i] = src[i];
}

// Bilinear footprint of one sample: the top-left corner, the fractional
// parts, and which of the two rows / two columns lie inside the image (a
// corner outside [0,H)x[0,W) has value 0: zero-extended image).
struct Footprint {
    float lh, lw;            // loc - floor(loc)
    bool r0, r1, c0, c1;     // rows h0, h0+1 and columns w0, w0+1 inside the image
    unsigned off;            // byte offset of corner (h0, w0) plus the channel offset
};

__device__ __forceinline__ bool footprint(const KArgs &a, int n, int ho, int wo, int k,
                                          float dx, float dy, int es, int chan_off, Footprint &f)
{
    const int kk = k + ((a.rc && k >= a.kc) ? 1 : 0);
    const int i = kk / a.kh, j = kk - i * a.kh;
    const float loc_w = __builtin_fmaf(a.scale, dx, (float)(wo * a.sw - a.pw + i * a.dw));
    const float loc_h = __builtin_fmaf(a.scale, dy, (float)(ho * a.sh - a.ph + j * a.dh));
    if (!(loc_h >= -1.0f && loc_h < (float)a.H && loc_w >= -1.0f && loc_w < (float)a.W))
        return false;   // all four corners outside (or NaN): the sample adds nothing
    const float fh = floorf(loc_h), fw = floorf(loc_w);
    const int h0 = (int)fh, w0 = (int)fw;
    f.lh = loc_h - fh;
    f.lw = loc_w - fw;
    f.r0 = h0 >= 0;
    f.r1 = h0 + 1 < a.H;
    f.c0 = w0 >= 0;
    f.c1 = w0 + 1 < a.W;
    // Negative offsets (row -1 of image 0) wrap to huge unsigned values and
    // fail the buffer range check like offsets past the end.
    f.off = ((unsigned)(n * a.H + h0) * (unsigned)a.W + (unsigned)w0) * (unsigned)(a.C * es) + (unsigned)chan_off;
    return true;
}

// Corner weights m*w_q with corners outside the image set to 0 (the loads of
// such corners return neighbouring or zero data, multiplied by 0; values are
// finite by contract).
__device__ __forceinline__ void corner_weights(const Footprint &f, float m, float &w00, float &w01,
                                               float &w10, float &w11)
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

// ---- forward -------------------------------------------------------------

template <typename T, int DP>
__global__ __launch_bounds__(256) void dcnv4_fwd_kernel(KArgs a)
{
    extern __shared__ u32x4 smem[];
    constexpr int NV = DP * (int)sizeof(T) / 16;   // 128-bit vectors per corner
    const int tile = xcd_tile(blockIdx.x, gridDim.x);
    const int pix0 = tile * a.pix_per_block;
    const int npix = min(a.pix_per_block, a.total_pix - pix0);
    stage_rows<T>(a, pix0, npix, smem);
    __syncthreads();

    const int gl = a.G * a.lanes;
    const int lp = threadIdx.x / gl;
    if (lp >= npix)
        return;
    const int rr = threadIdx.x - lp * gl;
    const int g = rr / a.lanes;
    const int chunk = rr - g * a.lanes;
    const int pix = pix0 + lp;
    const int wo = pix % a.Wo;
    const int t = pix / a.Wo;
    const int ho = t % a.Ho;
    const int n = t / a.Ho;
    const int es = (int)sizeof(T);
    const int chan_off = (g * a.Cg + chunk * DP) * es;
    const unsigned cs = (unsigned)(a.C * es), rs = (unsigned)a.W * cs;
    const T *om = reinterpret_cast<const T *>(smem) + lp * a.P + g * 3 * a.K;
    const __amdgpu_buffer_rsrc_t vr =
        __builtin_amdgcn_make_buffer_rsrc(const_cast<void *>(a.value), 0, a.value_bytes, kRawBufferConfig);

    float acc[DP];
#pragma unroll
    for (int c = 0; c < DP; ++c)
        acc[c] = 0.0f;

    for (int k = 0; k < a.K; ++k) {
        const float dx = Store<T>::scalar(om[2 * k]);
        const float dy = Store<T>::scalar(om[2 * k + 1]);
        const float m = Store<T>::scalar(om[2 * a.K + k]);
        Footprint f;
        if (!footprint(a, n, ho, wo, k, dx, dy, es, chan_off, f))
            continue;
        float w00, w01, w10, w11;
        corner_weights(f, m, w00, w01, w10, w11);
        u32x4 v00[NV], v01[NV], v10[NV], v11[NV];
#pragma unroll
        for (int v = 0; v < NV; ++v) {
            v00[v] = __builtin_amdgcn_raw_buffer_load_b128(vr, f.off + 16 * v, 0, 0);
            v01[v] = __builtin_amdgcn_raw_buffer_load_b128(vr, f.off + cs + 16 * v, 0, 0);
            v10[v] = __builtin_amdgcn_raw_buffer_load_b128(vr, f.off + rs + 16 * v, 0, 0);
            v11[v] = __builtin_amdgcn_raw_buffer_load_b128(vr, f.off + rs + cs + 16 * v, 0, 0);
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
    u32x4 *dst = reinterpret_cast<u32x4 *>(static_cast<T *>(a.out) + (size_t)pix * a.C + g * a.Cg + chunk * DP);
#pragma unroll
    for (int v = 0; v < NV; ++v)
        dst[v] = res[v];
}

// ---- backward (fp32) -----------------------------------------------------

__global__ __launch_bounds__(256) void dcnv4_zero_kernel(u32x4 *p, size_t nvec)
{
    const u32x4 z = {0u, 0u, 0u, 0u};
    for (size_t i = (size_t)blockIdx.x * blockDim.x + threadIdx.x; i < nvec; i += (size_t)gridDim.x * blockDim.x)
        p[i] = z;
}

template <int DP>
__global__ __launch_bounds__(256) void dcnv4_bwd_kernel(KArgs a)
{
    extern __shared__ u32x4 smem[];
    constexpr int NV = DP / 4;
    const int tile = xcd_tile(blockIdx.x, gridDim.x);
    const int pix0 = tile * a.pix_per_block;
    const int npix = min(a.pix_per_block, a.total_pix - pix0);
    float *s_om = reinterpret_cast<float *>(smem);
    float *s_grad = s_om + a.pix_per_block * a.P;
    stage_rows<float>(a, pix0, npix, smem);
    for (int i = threadIdx.x; i < npix * a.P; i += blockDim.x)
        s_grad[i] = 0.0f;
    __syncthreads();

    const int gl = a.G * a.lanes;
    const int lp = threadIdx.x / gl;
    if (lp < npix) {
        const int rr = threadIdx.x - lp * gl;
        const int g = rr / a.lanes;
        const int chunk = rr - g * a.lanes;
        const int pix = pix0 + lp;
        const int wo = pix % a.Wo;
        const int t = pix / a.Wo;
        const int ho = t % a.Ho;
        const int n = t / a.Ho;
        const int chan_off = (g * a.Cg + chunk * DP) * 4;
        const unsigned cs = (unsigned)(a.C * 4), rs = (unsigned)a.W * cs;
        const float *om = s_om + lp * a.P + g * 3 * a.K;
        float *gomr = s_grad + lp * a.P + g * 3 * a.K;
        const __amdgpu_buffer_rsrc_t vr =
            __builtin_amdgcn_make_buffer_rsrc(const_cast<void *>(a.value), 0, a.value_bytes, kRawBufferConfig);
        const __amdgpu_buffer_rsrc_t gr =
            __builtin_amdgcn_make_buffer_rsrc(a.gvalue, 0, a.value_bytes, kRawBufferConfig);

        float go[DP];
        {
            const u32x4 *src = reinterpret_cast<const u32x4 *>(a.gout + (size_t)pix * a.C + g * a.Cg + chunk * DP);
#pragma unroll
            for (int v = 0; v < NV; ++v) {
                const f32x4 r = __builtin_bit_cast(f32x4, src[v]);
                for (int e = 0; e < 4; ++e)
                    go[4 * v + e] = r[e];
            }
        }

        for (int k = 0; k < a.K; ++k) {
            const float dx = om[2 * k], dy = om[2 * k + 1], m = om[2 * a.K + k];
            Footprint f;
            float gm = 0.0f, gw = 0.0f, gh = 0.0f;
            const bool live = footprint(a, n, ho, wo, k, dx, dy, 4, chan_off, f);
            if (live) {
                u32x4 v00[NV], v01[NV], v10[NV], v11[NV];
#pragma unroll
                for (int v = 0; v < NV; ++v) {
                    v00[v] = __builtin_amdgcn_raw_buffer_load_b128(vr, f.off + 16 * v, 0, 0);
                    v01[v] = __builtin_amdgcn_raw_buffer_load_b128(vr, f.off + cs + 16 * v, 0, 0);
                    v10[v] = __builtin_amdgcn_raw_buffer_load_b128(vr, f.off + rs + 16 * v, 0, 0);
                    v11[v] = __builtin_amdgcn_raw_buffer_load_b128(vr, f.off + rs + cs + 16 * v, 0, 0);
                }
                // t_q = sum_c grad_out_c * v_q,c : every gradient of the
                // sample is a fixed combination of the four corner dots.
                float t00 = 0.0f, t01 = 0.0f, t10 = 0.0f, t11 = 0.0f;
#pragma unroll
                for (int c = 0; c < DP; ++c) {
                    t00 = __builtin_fmaf(go[c], Store<float>::get(v00, c), t00);
                    t01 = __builtin_fmaf(go[c], Store<float>::get(v01, c), t01);
                    t10 = __builtin_fmaf(go[c], Store<float>::get(v10, c), t10);
                    t11 = __builtin_fmaf(go[c], Store<float>::get(v11, c), t11);
                }
                // Zero-extended image: dots of corners outside are 0.
                const bool q00 = f.r0 && f.c0, q01 = f.r0 && f.c1, q10 = f.r1 && f.c0, q11 = f.r1 && f.c1;
                t00 = q00 ? t00 : 0.0f;
                t01 = q01 ? t01 : 0.0f;
                t10 = q10 ? t10 : 0.0f;
                t11 = q11 ? t11 : 0.0f;
                const float lh = f.lh, lw = f.lw, hh = 1.0f - lh, hw = 1.0f - lw;
                // d/dm: the sample; d/d loc_w and d/d loc_h of the bilinear
                // sample inside the cell chosen by floor (right derivative).
                gm = hh * (hw * t00 + lw * t01) + lh * (hw * t10 + lw * t11);
                gw = hh * (t01 - t00) + lh * (t11 - t10);
                gh = hw * (t10 - t00) + lw * (t11 - t01);
                // grad_value: m * w_q * grad_out_c to each corner; corners
                // outside the image get a zero weight, and those outside the
                // tensor are dropped by the buffer range check.
                float w00, w01, w10, w11;
                corner_weights(f, m, w00, w01, w10, w11);
#pragma unroll
                for (int c = 0; c < DP; ++c) {
                    const unsigned o = f.off + 4 * c;
                    buffer_atomic_fadd(w00 * go[c], gr, o, 0, 0);
                    buffer_atomic_fadd(w01 * go[c], gr, o + cs, 0, 0);
                    buffer_atomic_fadd(w10 * go[c], gr, o + rs, 0, 0);
                    buffer_atomic_fadd(w11 * go[c], gr, o + rs + cs, 0, 0);
                }
            }
            // reduce the partial sums of the lanes sharing this (pixel, group);
            // they are consecutive and aligned, so xor-butterflies stay inside
            for (int d = 1; d < a.lanes; d <<= 1) {
                gm += __shfl_xor(gm, d);
                gw += __shfl_xor(gw, d);
                gh += __shfl_xor(gh, d);
            }
            if (chunk == 0) {
                const float sm = a.scale * m;
                gomr[2 * k] = sm * gw;
                gomr[2 * k + 1] = sm * gh;
                gomr[2 * a.K + k] = gm;
            }
        }
    }
    __syncthreads();
    // grad_offset_mask rows of this block (padding stays 0)
    {
        u32x4 *dst = reinterpret_cast<u32x4 *>(a.gom + (size_t)pix0 * a.P);
        const u32x4 *src = reinterpret_cast<const u32x4 *>(s_grad);
        const int nvec = npix * a.P / 4;
        for (int i = threadIdx.x; i < nvec; i += blockDim.x)
            dst[i] = src[i];
    }
}

template <typename T>
hipError_t launch_fwd_t(const Problem &p, const Plan &plan, const KArgs &a, int blocks, hipStream_t s)
{
    switch (plan.dp) {
    case 16:
        hipLaunchKernelGGL((dcnv4_fwd_kernel<T, 16>), dim3(blocks), dim3(plan.threads), plan.lds_bytes, s, a);
        break;
    case 8:
        hipLaunchKernelGGL((dcnv4_fwd_kernel<T, 8>), dim3(blocks), dim3(plan.threads), plan.lds_bytes, s, a);
        break;
    case 4:
        if constexpr (sizeof(T) == 4) {
            hipLaunchKernelGGL((dcnv4_fwd_kernel<T, 4>), dim3(blocks), dim3(plan.threads), plan.lds_bytes, s, a);
            break;
        }
        return hipErrorInvalidValue;
    default:
        return hipErrorInvalidValue;
    }
    (void)p;
    return hipGetLastError();
}

KArgs make_args(const Problem &p, const Plan &plan)
{
    KArgs a{};
    a.H = p.H;
    a.W = p.W;
    a.Ho = p.Ho;
    a.Wo = p.Wo;
    a.G = p.G;
    a.Cg = p.Cg;
    a.C = p.C;
    a.K = p.K;
    a.P = p.P;
    a.kh = p.kh;
    a.sh = p.sh;
    a.sw = p.sw;
    a.ph = p.ph;
    a.pw = p.pw;
    a.dh = p.dh;
    a.dw = p.dw;
    a.rc = p.remove_center;
    a.kc = ((p.kw - 1) / 2) * p.kh + (p.kh - 1) / 2;
    a.scale = p.offset_scale;
    a.lanes = plan.lanes;
    a.pix_per_block = plan.pix_per_block;
    a.total_pix = p.N * p.Ho * p.Wo;
    a.value_bytes = p.N * p.H * p.W * p.C * p.elem;
    return a;
}

}  // namespace

hipError_t launch_forward(const Problem &p, const Plan &plan, const void *value, const void *offset_mask,
                          void *output, hipStream_t stream)
{
    KArgs a = make_args(p, plan);
    a.value = value;
    a.om = offset_mask;
    a.out = output;
    const int blocks = (a.total_pix + plan.pix_per_block - 1) / plan.pix_per_block;
    switch (p.dtype) {
    case 0:
        return launch_fwd_t<float>(p, plan, a, blocks, stream);
    case 1:
        return launch_fwd_t<_Float16>(p, plan, a, blocks, stream);
    case 2:
        return launch_fwd_t<bf16_t>(p, plan, a, blocks, stream);
    default:
        return hipErrorInvalidValue;
    }
}

hipError_t launch_backward(const Problem &p, const Plan &plan, const void *value, const void *offset_mask,
                           const void *grad_output, void *grad_value, void *grad_offset_mask,
                           hipStream_t stream)
{
    KArgs a = make_args(p, plan);
    a.value = value;
    a.om = offset_mask;
    a.gout = static_cast<const float *>(grad_output);
    a.gvalue = static_cast<float *>(grad_value);
    a.gom = static_cast<float *>(grad_offset_mask);
    const size_t nvec = (size_t)a.value_bytes / 16;
    const int zblocks = (int)std::min<size_t>((nvec + 255) / 256, 4096);
    hipLaunchKernelGGL(dcnv4_zero_kernel, dim3(zblocks), dim3(256), 0, stream,
                       static_cast<u32x4 *>(grad_value), nvec);
    hipError_t e = hipGetLastError();
    if (e != hipSuccess)
        return e;
    const int blocks = (a.total_pix + plan.pix_per_block - 1) / plan.pix_per_block;
    switch (plan.dp) {
    case 4:
        hipLaunchKernelGGL((dcnv4_bwd_kernel<4>), dim3(blocks), dim3(plan.threads), plan.lds_bytes, stream, a);
        break;
    case 8:
        hipLaunchKernelGGL((dcnv4_bwd_kernel<8>), dim3(blocks), dim3(plan.threads), plan.lds_bytes, stream, a);
        break;
    case 16:
        hipLaunchKernelGGL((dcnv4_bwd_kernel<16>), dim3(blocks), dim3(plan.threads), plan.lds_bytes, stream, a);
        break;
    default:
        return hipErrorInvalidValue;
    }
    return hipGetLastError();
}

}  // namespace dcnv4
