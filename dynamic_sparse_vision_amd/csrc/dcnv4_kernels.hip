// General-path HIP kernels of the DCNv4 spatial aggregation (gfx950).
//
// Operation ("Efficient Deformable ConvNets", DCNv3 recap equation of the
// CSDN walkthrough "DCNv4论文解析", section 1.2, without the softmax of
// section 2.1): for each output pixel, group g and grid point k, a bilinear
// sample of the channel-last value tensor at
//   (ho*stride_h - pad_h + j*dil_h + s*dy,  wo*stride_w - pad_w + i*dil_w + s*dx)
// with zero padding, times an unnormalised scalar m, summed over k.
//
// These kernels handle any validated shape: one thread owns DP contiguous
// channels of one (pixel, group) (walkthrough section 2.2: offsets, masks and
// bilinear coefficients read/computed once per D' channels), the block's
// offset/mask rows are staged in LDS (blog "DCNv4架构解析", section
// "并行计算架构设计"), corners are 128-bit raw buffer loads whose range check
// returns 0 outside the tensor, and grad_value is summed with device atomics.
// The tiled kernels (dcnv4_tiled_*.hip) are used where their LDS budget fits.

#include "dcnv4_device.h"
#include "dcnv4_internal.h"

#include <algorithm>

namespace dcnv4 {
namespace {

using namespace dev;

struct KArgs {
    Geom geo;
    const void *value;
    const void *om;
    void *out;            // forward output
    const float *gout;    // backward: grad_output
    float *gvalue;        // backward: grad_value
    float *gom;           // backward: grad_offset_mask
    int G, Cg, K, P;
    int lanes, pix_per_block, total_pix;
    int value_bytes;      // bytes of value (and of grad_value) in this launch
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

template <typename T, int DP>
__global__ __launch_bounds__(256) void dcnv4_fwd_general(KArgs a)
{
    extern __shared__ u32x4 smem[];
    constexpr int NV = DP * (int)sizeof(T) / 16;   // 128-bit vectors per corner
    const Geom &geo = a.geo;
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
    const int wo = pix % geo.Wo;
    const int t = pix / geo.Wo;
    const int ho = t % geo.Ho;
    const int n = t / geo.Ho;
    const int es = (int)sizeof(T);
    const int chan_off = (g * a.Cg + chunk * DP) * es;
    const unsigned cs = (unsigned)(geo.C * es), rs = (unsigned)geo.W * cs;
    const T *om = reinterpret_cast<const T *>(smem) + lp * a.P + g * 3 * a.K;
    const __amdgpu_buffer_rsrc_t vr = rsrc(a.value, a.value_bytes);

    float acc[DP];
#pragma unroll
    for (int c = 0; c < DP; ++c)
        acc[c] = 0.0f;

    for (int k = 0; k < a.K; ++k) {
        const float dx = Store<T>::scalar(om[2 * k]);
        const float dy = Store<T>::scalar(om[2 * k + 1]);
        const float m = Store<T>::scalar(om[2 * a.K + k]);
        const Loc l = locate(geo, ho, wo, k, dx, dy);
        if (!live(geo, l))
            continue;
        const Footprint f = footprint(geo, l);
        const unsigned off = corner_offset(geo, n, f, es, chan_off);
        float w00, w01, w10, w11;
        masked_weights(f, m, w00, w01, w10, w11);
        u32x4 v00[NV], v01[NV], v10[NV], v11[NV];
#pragma unroll
        for (int v = 0; v < NV; ++v) {
            v00[v] = load16(vr, off + 16 * v);
            v01[v] = load16(vr, off + cs + 16 * v);
            v10[v] = load16(vr, off + rs + 16 * v);
            v11[v] = load16(vr, off + rs + cs + 16 * v);
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
    u32x4 *dst = reinterpret_cast<u32x4 *>(static_cast<T *>(a.out) + (size_t)pix * geo.C + g * a.Cg + chunk * DP);
#pragma unroll
    for (int v = 0; v < NV; ++v)
        dst[v] = res[v];
}

__global__ __launch_bounds__(256) void dcnv4_zero_kernel(u32x4 *p, size_t nvec)
{
    const u32x4 z = {0u, 0u, 0u, 0u};
    for (size_t i = (size_t)blockIdx.x * blockDim.x + threadIdx.x; i < nvec; i += (size_t)gridDim.x * blockDim.x)
        p[i] = z;
}

template <int DP>
__global__ __launch_bounds__(256) void dcnv4_bwd_general(KArgs a)
{
    extern __shared__ u32x4 smem[];
    constexpr int NV = DP / 4;
    const Geom &geo = a.geo;
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
        const int wo = pix % geo.Wo;
        const int t = pix / geo.Wo;
        const int ho = t % geo.Ho;
        const int n = t / geo.Ho;
        const int chan_off = (g * a.Cg + chunk * DP) * 4;
        const unsigned cs = (unsigned)(geo.C * 4), rs = (unsigned)geo.W * cs;
        const float *om = s_om + lp * a.P + g * 3 * a.K;
        float *gomr = s_grad + lp * a.P + g * 3 * a.K;
        const __amdgpu_buffer_rsrc_t vr = rsrc(a.value, a.value_bytes);
        const __amdgpu_buffer_rsrc_t gr = rsrc(a.gvalue, a.value_bytes);

        float go[DP];
        {
            const u32x4 *src = reinterpret_cast<const u32x4 *>(a.gout + (size_t)pix * geo.C + g * a.Cg + chunk * DP);
#pragma unroll
            for (int v = 0; v < NV; ++v) {
                const f32x4 r = __builtin_bit_cast(f32x4, src[v]);
                for (int e = 0; e < 4; ++e)
                    go[4 * v + e] = r[e];
            }
        }

        for (int k = 0; k < a.K; ++k) {
            const float dx = om[2 * k], dy = om[2 * k + 1], m = om[2 * a.K + k];
            float gm = 0.0f, gw = 0.0f, gh = 0.0f;
            const Loc l = locate(geo, ho, wo, k, dx, dy);
            if (live(geo, l)) {
                const Footprint f = footprint(geo, l);
                const unsigned off = corner_offset(geo, n, f, 4, chan_off);
                u32x4 v00[NV], v01[NV], v10[NV], v11[NV];
#pragma unroll
                for (int v = 0; v < NV; ++v) {
                    v00[v] = load16(vr, off + 16 * v);
                    v01[v] = load16(vr, off + cs + 16 * v);
                    v10[v] = load16(vr, off + rs + 16 * v);
                    v11[v] = load16(vr, off + rs + cs + 16 * v);
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
                t00 = (f.r0 && f.c0) ? t00 : 0.0f;
                t01 = (f.r0 && f.c1) ? t01 : 0.0f;
                t10 = (f.r1 && f.c0) ? t10 : 0.0f;
                t11 = (f.r1 && f.c1) ? t11 : 0.0f;
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
                masked_weights(f, m, w00, w01, w10, w11);
#pragma unroll
                for (int c = 0; c < DP; ++c) {
                    const unsigned o = off + 4 * c;
                    dcnv4_buffer_atomic_fadd(w00 * go[c], gr, o, 0, 0);
                    dcnv4_buffer_atomic_fadd(w01 * go[c], gr, o + cs, 0, 0);
                    dcnv4_buffer_atomic_fadd(w10 * go[c], gr, o + rs, 0, 0);
                    dcnv4_buffer_atomic_fadd(w11 * go[c], gr, o + rs + cs, 0, 0);
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
                const float sm = geo.scale * m;
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
hipError_t launch_fwd_t(const Plan &plan, const KArgs &a, int blocks, hipStream_t s)
{
    switch (plan.dp) {
    case 16:
        hipLaunchKernelGGL((dcnv4_fwd_general<T, 16>), dim3(blocks), dim3(plan.threads), plan.lds_bytes, s, a);
        break;
    case 8:
        hipLaunchKernelGGL((dcnv4_fwd_general<T, 8>), dim3(blocks), dim3(plan.threads), plan.lds_bytes, s, a);
        break;
    case 4:
        if constexpr (sizeof(T) == 4) {
            hipLaunchKernelGGL((dcnv4_fwd_general<T, 4>), dim3(blocks), dim3(plan.threads), plan.lds_bytes, s, a);
            break;
        }
        return hipErrorInvalidValue;
    default:
        return hipErrorInvalidValue;
    }
    return hipGetLastError();
}

KArgs make_args(const Problem &p, const Plan &plan)
{
    KArgs a{};
    a.geo = make_geom(p);
    a.G = p.G;
    a.Cg = p.Cg;
    a.K = p.K;
    a.P = p.P;
    a.lanes = plan.lanes;
    a.pix_per_block = plan.pix_per_block;
    a.total_pix = p.N * p.Ho * p.Wo;
    a.value_bytes = p.N * p.H * p.W * p.C * p.elem;
    return a;
}

}  // namespace

dev::Geom make_geom(const Problem &p)
{
    dev::Geom g{};
    g.H = p.H;
    g.W = p.W;
    g.C = p.C;
    g.Ho = p.Ho;
    g.Wo = p.Wo;
    g.kh = p.kh;
    g.kw = p.kw;
    g.sh = p.sh;
    g.sw = p.sw;
    g.ph = p.ph;
    g.pw = p.pw;
    g.dh = p.dh;
    g.dw = p.dw;
    g.rc = p.remove_center;
    g.kc = ((p.kw - 1) / 2) * p.kh + (p.kh - 1) / 2;
    g.scale = p.offset_scale;
    return g;
}

hipError_t launch_zero(void *p, size_t bytes, hipStream_t stream)
{
    const size_t nvec = bytes / 16;
    const int blocks = (int)std::min<size_t>((nvec + 255) / 256, 4096);
    if (blocks == 0)
        return hipSuccess;
    hipLaunchKernelGGL(dcnv4_zero_kernel, dim3(blocks), dim3(256), 0, stream, static_cast<u32x4 *>(p), nvec);
    return hipGetLastError();
}

hipError_t launch_forward_general(const Problem &p, const Plan &plan, const void *value, const void *offset_mask,
                                  void *output, hipStream_t stream)
{
    KArgs a = make_args(p, plan);
    a.value = value;
    a.om = offset_mask;
    a.out = output;
    const int blocks = (a.total_pix + plan.pix_per_block - 1) / plan.pix_per_block;
    switch (p.dtype) {
    case 0:
        return launch_fwd_t<float>(plan, a, blocks, stream);
    case 1:
        return launch_fwd_t<_Float16>(plan, a, blocks, stream);
    case 2:
        return launch_fwd_t<bf16_t>(plan, a, blocks, stream);
    default:
        return hipErrorInvalidValue;
    }
}

hipError_t launch_backward_general(const Problem &p, const Plan &plan, const void *value, const void *offset_mask,
                                   const void *grad_output, void *grad_value, void *grad_offset_mask,
                                   hipStream_t stream)
{
    KArgs a = make_args(p, plan);
    a.value = value;
    a.om = offset_mask;
    a.gout = static_cast<const float *>(grad_output);
    a.gvalue = static_cast<float *>(grad_value);
    a.gom = static_cast<float *>(grad_offset_mask);
    hipError_t e = launch_zero(grad_value, (size_t)a.value_bytes, stream);
    if (e != hipSuccess)
        return e;
    const int blocks = (a.total_pix + plan.pix_per_block - 1) / plan.pix_per_block;
    switch (plan.dp) {
    case 4:
        hipLaunchKernelGGL((dcnv4_bwd_general<4>), dim3(blocks), dim3(plan.threads), plan.lds_bytes, stream, a);
        break;
    case 8:
        hipLaunchKernelGGL((dcnv4_bwd_general<8>), dim3(blocks), dim3(plan.threads), plan.lds_bytes, stream, a);
        break;
    case 16:
        hipLaunchKernelGGL((dcnv4_bwd_general<16>), dim3(blocks), dim3(plan.threads), plan.lds_bytes, stream, a);
        break;
    default:
        return hipErrorInvalidValue;
    }
    return hipGetLastError();
}

}  // namespace dcnv4
