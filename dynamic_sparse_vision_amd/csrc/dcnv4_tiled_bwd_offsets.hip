// Backward grad_offset_mask kernel of the LDS-tiled DCNv4 path (shared pieces: dcnv4_tiled.h).

#include "dcnv4.h"
#include "dcnv4_tiled.h"

namespace dcnv4 {
namespace tiled {
namespace {

typedef _Float16 f16x2 __attribute__((ext_vector_type(2)));
typedef __bf16 bf16x2 __attribute__((ext_vector_type(2)));

// sum_c grad_out_c * v_c over a lane's channels (NV 16-byte vectors of each).
// 16-bit storage: one dot2 instruction per pair of channels (the product of
// two 16-bit numbers is exact in fp32, the sum is accumulated in fp32);
// fp32: one FMA per channel, in channel order.
template <typename T, int NV>
__device__ __forceinline__ float corner_dot(const u32x4 (&go)[NV], const u32x4 (&v)[NV])
{
    float t = 0.0f;
#pragma unroll
    for (int i = 0; i < NV; ++i) {
#pragma unroll
        for (int e = 0; e < 4; ++e) {
            const unsigned x = go[i][e], y = v[i][e];
            if constexpr (sizeof(T) == 4)
                t = __builtin_fmaf(__builtin_bit_cast(float, x), __builtin_bit_cast(float, y), t);
            else if constexpr (__is_same(T, _Float16))
                t = __builtin_amdgcn_fdot2(__builtin_bit_cast(f16x2, x), __builtin_bit_cast(f16x2, y), t, false);
            else
                t = __builtin_amdgcn_fdot2_f32_bf16(__builtin_bit_cast(bf16x2, x), __builtin_bit_cast(bf16x2, y), t,
                                                    false);
        }
    }
    return t;
}

// Blocks as the forward's: a th x tw output tile of one image and gb groups,
// `lanes` threads of DP channels per pixel and group, the region's value
// rows staged in LDS while each lane loads its pixel's offsets, masks and
// grad_output channels.  Per sample, the dot products t_q = sum_c
// grad_out_c * v_q,c of the four corners give d/dm and d/d(loc) (right
// derivative at integers), summed over the pixel's lanes; the K samples are
// one straight-line loop (KMAX >= K) whose gradients stay in registers.  A
// sample whose footprint lies in the region reads its corners from LDS; a
// live one that does not is taken after the loop from global memory.
//
// grad_value: the cell-tile kernel has written every cell with the
// contributions of the samples within Rc of their grid position (|floor(loc)
// - grid position| <= Rc on both axes, the same test in the same fp32
// arithmetic there).  Every other live sample is added here with device
// atomics at the end, one instruction per sample and up to 16 channels of
// all four corners, issued by the whole wave.
//
// At the end the region's LDS holds the tile's gradient rows (fp32, each
// pixel's gb groups contiguous as in offset_mask), written back with
// coalesced dword stores.
template <typename T, int DP, int KMAX, bool SM>
__global__ __launch_bounds__(kMaxTileThreads) __attribute__((amdgpu_waves_per_eu(KMAX <= 9 ? 4 : 1))) void dcnv4_bwd_offsets_tiled(TArgs a)
{
    extern __shared__ u32x4 smem[];
    constexpr int es = (int)sizeof(T);
    constexpr int NV = DP * es / 16;
    constexpr int EPV = 16 / es;
    constexpr int NVO = (2 * KMAX + 2 * (EPV - 1)) / EPV;
    constexpr int NVM = (KMAX + 2 * (EPV - 1)) / EPV;
    const Geom &geo = a.geo;
    const Tile t = block_tile(a);
    const Region rg = tile_region(a, t);
    char *lds = reinterpret_cast<char *>(smem);
    stage_region(a, t, rg, lds, es);

    const int per_pixel_shift = a.lanes_shift + a.gb_shift;
    const int q = threadIdx.x >> per_pixel_shift;
    const int r_in = threadIdx.x & ((1 << per_pixel_shift) - 1);
    const int gl = r_in >> a.lanes_shift;   // group within the block
    const int chunk = r_in & ((1 << a.lanes_shift) - 1);
    const int lanes = 1 << a.lanes_shift;
    const int g = t.g + gl;
    const int py = (int)divm((unsigned)q, a.tw_magic);
    const int px = q - py * a.tw;
    const int oy = t.oy0 + py, ox = t.ox0 + px;
    const bool valid = py < a.th && oy < geo.Ho && ox < geo.Wo;
    const unsigned pix = (unsigned)((t.n * geo.Ho + oy) * geo.Wo + ox);
    // offsets and masks: aligned vectors from the one holding the group's
    // first entry, shifted with bit masks (the shift differs between the
    // groups of a wave); grad_output: the lane's DP channels
    const int eo = g * 3 * a.K, em = eo + 2 * a.K;
    const int mis_o = eo & (EPV - 1), mis_m = em & (EPV - 1);
    const unsigned om_row = pix * (unsigned)(a.P * es) + (unsigned)(eo * es);
    u32x4 vov[NVO], vmv[NVM], gov[NV];
    {
        const __amdgpu_buffer_rsrc_t omr = rsrc(a.om, a.om_bytes);
        const unsigned row = valid ? pix * (unsigned)(a.P * es) : kOutOfRange;
        const unsigned bo = (unsigned)((eo - mis_o) * es), bm = (unsigned)((em - mis_m) * es);
#pragma unroll
        for (int j = 0; j < NVO; ++j)
            vov[j] = load16(omr, row == kOutOfRange ? kOutOfRange : row + bo + 16u * j);
#pragma unroll
        for (int j = 0; j < NVM; ++j)
            vmv[j] = load16(omr, row == kOutOfRange ? kOutOfRange : row + bm + 16u * j);
        const __amdgpu_buffer_rsrc_t gor = rsrc(a.gout, a.gout_bytes);
        const unsigned gch =
            valid ? pix * (unsigned)(geo.C * es) + (unsigned)((g * a.Cg + chunk * DP) * es) : kOutOfRange;
#pragma unroll
        for (int v = 0; v < NV; ++v)
            gov[v] = load16(gor, gch == kOutOfRange ? kOutOfRange : gch + 16u * v);
    }
    // the grid table, uniform: for up to 9 points loaded once, outside the
    // sample loop (25 points would crowd the scalar registers; they are
    // read where used)
    constexpr int KG = KMAX <= 9 ? KMAX : 1;
    float gdh_r[KG], gdw_r[KG];
#pragma unroll
    for (int k = 0; k < KG; ++k) {
        gdh_r[k] = a.gdh[k];
        gdw_r[k] = a.gdw[k];
    }
    auto gdh = [&](int k) { return KMAX <= 9 ? gdh_r[k < KG ? k : 0] : a.gdh[k]; };
    auto gdw = [&](int k) { return KMAX <= 9 ? gdw_r[k < KG ? k : 0] : a.gdw[k]; };
    staging_done();

    float offs[2 * KMAX], msk[KMAX];
    entries_of<T>(vov, mis_o, offs);
    entries_of<T>(vmv, mis_m, msk);
    float sm_max = 0.0f, sm_inv = 1.0f;
    if (SM) {
        // msk becomes the probabilities p_k = exp(m_k - sm_max) * sm_inv
        sm_max = msk[0];
#pragma unroll
        for (int k = 1; k < KMAX; ++k)
            sm_max = k < a.K ? fmaxf(sm_max, msk[k]) : sm_max;
        float sum = 0.0f;
#pragma unroll
        for (int k = 0; k < KMAX; ++k) {
            msk[k] = k < a.K ? expf(msk[k] - sm_max) : 0.0f;
            sum += msk[k];
        }
        sm_inv = 1.0f / sum;
#pragma unroll
        for (int k = 0; k < KMAX; ++k)
            msk[k] *= sm_inv;
    }
    const float bh0 = (float)(oy * geo.sh - geo.ph), bw0 = (float)(ox * geo.sw - geo.pw);
    // footprints (fh, fw) .. (fh + 1, fw + 1) inside the region
    const float lo_h = (float)rg.y0, hi_h = (float)(rg.y0 + rg.rows - 2);
    const float lo_w = (float)rg.x0, hi_w = (float)(rg.x0 + rg.cols - 2);
    const unsigned colb = (unsigned)a.pst * 16u, rowb = (unsigned)a.rw * colb;
    const unsigned abias = 0u - (unsigned)rg.y0 * rowb - (unsigned)rg.x0 * colb - (1u << 22) * (rowb + colb);
    const char *vb = lds + (gl * a.nvp + chunk * NV) * 16;   // this lane's vectors in a pixel's slice
    const float Hf = (float)geo.H, Wf = (float)geo.W, Rcf = (float)a.Rc;

    // gradients: d/d(dx_k), d/d(dy_k), d/dm_k (d/dp_k in softmax mode until the end)
    float gx[KMAX], gy[KMAX], gmk[KMAX];
    unsigned glob = 0;   // live samples outside the region: corners from global memory
    unsigned atom = 0;   // live samples beyond Rc: grad_value by device atomics
    // Keeps the loop in program order: sample k's gradients are complete
    // here and no LDS read moves across, and sample k + 1's inputs pass
    // through it, so its placement is not computed ahead (left alone, the
    // compiler issues every sample's reads first and runs out of registers).
    auto fence = [&](int k) {
        asm volatile("" : "+v"(gx[k]), "+v"(gy[k]), "+v"(gmk[k])::"memory");
        if (k + 1 < KMAX)
            asm volatile("" : "+v"(offs[2 * k + 2]), "+v"(offs[2 * k + 3]), "+v"(msk[k + 1]));
    };
#pragma unroll
    for (int k = 0; k < KMAX; ++k) {
        const bool in_k = valid && k < a.K;
        const float bh = bh0 + gdh(k), bw = bw0 + gdw(k);
        const float lh = __builtin_fmaf(geo.scale, offs[2 * k + 1], bh);
        const float lw = __builtin_fmaf(geo.scale, offs[2 * k], bw);
        const float fh = __builtin_floorf(lh), fw = __builtin_floorf(lw);
        // each test is false for NaN; huge and infinite coordinates fail too
        const bool nr = in_k && fh >= lo_h && fh <= hi_h && fw >= lo_w && fw <= hi_w;
        const bool live = in_k && lh >= -1.0f && lh < Hf && lw >= -1.0f && lw < Wf;
        const bool cell = __builtin_fabsf(fh - bh) <= Rcf && __builtin_fabsf(fw - bw) <= Rcf;
        glob |= (!nr && live) ? (1u << k) : 0u;
        atom |= (!cell && live) ? (1u << k) : 0u;
        // floors become integers by bit pattern (defined for every float)
        const unsigned addr = __umul24(biased_int(fh), rowb) + __umul24(biased_int(fw), colb) + abias;
        const unsigned ad = nr ? addr : 0u;
        const float ah = nr ? lh - fh : 0.0f, aw = nr ? lw - fw : 0.0f;
        const u32x4 *q00 = reinterpret_cast<const u32x4 *>(vb + ad);
        const u32x4 *q01 = reinterpret_cast<const u32x4 *>(vb + ad + colb);
        const u32x4 *q10 = reinterpret_cast<const u32x4 *>(vb + ad + rowb);
        const u32x4 *q11 = reinterpret_cast<const u32x4 *>(vb + ad + rowb + colb);
        u32x4 v00[NV], v01[NV], v10[NV], v11[NV];
#pragma unroll
        for (int v = 0; v < NV; ++v) {
            v00[v] = q00[v];
            v01[v] = q01[v];
            v10[v] = q10[v];
            v11[v] = q11[v];
        }
        float gm, gw, gh;
        sample_grads(ah, aw, corner_dot<T>(gov, v00), corner_dot<T>(gov, v01), corner_dot<T>(gov, v10),
                     corner_dot<T>(gov, v11), gm, gw, gh);
        gm = pixel_sum(nr ? gm : 0.0f, lanes);
        gw = pixel_sum(nr ? gw : 0.0f, lanes);
        gh = pixel_sum(nr ? gh : 0.0f, lanes);
        const float sm = geo.scale * msk[k];
        gx[k] = sm * gw;
        gy[k] = sm * gh;
        gmk[k] = gm;
        fence(k);
    }
    __syncthreads();   // the value region is no longer read

    // the pixel's gradient row of its group, fp32, from float 3K * (q * gb + gl)
    float *grow = reinterpret_cast<float *>(lds) + (q * a.gb + gl) * 3 * a.K;
    const bool writer = valid && chunk == 0;
    if (writer) {
#pragma unroll
        for (int k = 0; k < KMAX; ++k) {
            if (k < a.K) {
                grow[2 * k] = gx[k];
                grow[2 * k + 1] = gy[k];
                grow[2 * a.K + k] = gmk[k];
            }
        }
    }
    // Samples the loop left out, in rounds: each lane takes its lowest
    // pending sample (the lanes of a pixel and group have the same bits, so
    // they take the same one and the pixel sums see them all active) and
    // loads its offsets and mask again (no register array is indexed by a
    // run-time k, and the entries need not stay live through the loop).
    //  - outside the region: corners from global memory; its gradients
    //    replace the zeros in the row;
    //  - beyond Rc: its grad_value contributions, by device atomics.  The
    //    lanes prepare their samples' weights and corner offset, then the
    //    wave adds them one sample at a time, lane l taking channel l % Cg of
    //    corner l / Cg (corners (h0, w0), (h0, w0 + 1), (h0 + 1, w0),
    //    (h0 + 1, w0 + 1); two instructions for Cg = 32).
    {
        const __amdgpu_buffer_rsrc_t omr = rsrc(a.om, a.om_bytes);
        auto entry = [&](int idx) -> float {
            if constexpr (es == 4)
                return __builtin_bit_cast(float,
                                          __builtin_amdgcn_raw_buffer_load_b32(omr, om_row + 4u * (unsigned)idx, 0, 0));
            else
                return Store<T>::from_bits(__builtin_amdgcn_raw_buffer_load_b16(omr, om_row + 2u * (unsigned)idx, 0, 0));
        };
        const __amdgpu_buffer_rsrc_t vr = rsrc(a.value, a.value_bytes);
        const __amdgpu_buffer_rsrc_t gr = rsrc(a.gvalue, a.gvalue_bytes);
        const int chan_off = (g * a.Cg + chunk * DP) * es;
        const unsigned cs = (unsigned)(geo.C * es), rs = (unsigned)geo.W * cs;
        const unsigned gcs = (unsigned)(geo.C * 4), grs = (unsigned)geo.W * gcs;
        const unsigned gv_base = (unsigned)(t.n * geo.H) * grs + (unsigned)(g * a.Cg * 4);
        const int lane = threadIdx.x & 63;
        const int my_c = lane & (a.Cg - 1), corner0 = lane >> a.cg_shift;
        const int per_instr = 64 >> a.cg_shift;   // corners per atomic instruction
        // where channel my_c of a pixel and group lives: lane my_lane of the
        // group's lanes, dword my_dw of its grad_output vectors
        const int my_lane = my_c / DP;
        const int my_dw = (my_c % DP) * es / 4;
        unsigned rest = glob | atom;
        while (__ballot(rest != 0u)) {
            const bool have = rest != 0u;
            const int k = have ? __builtin_ctz(rest) : 0;
            rest &= rest - 1u;
            const bool do_glob = have && ((glob >> k) & 1u), do_atom = have && ((atom >> k) & 1u);
            float w00 = 0.0f, w01 = 0.0f, w10 = 0.0f, w11 = 0.0f;
            unsigned cbase = 0u;
            if (have) {
                const float dx = entry(2 * k), dy = entry(2 * k + 1), m0 = entry(2 * a.K + k);
                const float m = SM ? expf(m0 - sm_max) * sm_inv : m0;
                int gi, gj;
                grid_point(geo, k, gi, gj);
                const float lh = __builtin_fmaf(geo.scale, dy, bh0 + (float)(gj * geo.dh));
                const float lw = __builtin_fmaf(geo.scale, dx, bw0 + (float)(gi * geo.dw));
                const float fh = __builtin_floorf(lh), fw = __builtin_floorf(lw);
                Footprint f;   // live: -1 <= floor < size, so the conversions are exact
                f.h0 = (int)fh;
                f.w0 = (int)fw;
                f.lh = lh - fh;
                f.lw = lw - fw;
                f.r0 = f.h0 >= 0;
                f.r1 = f.h0 + 1 < geo.H;
                f.c0 = f.w0 >= 0;
                f.c1 = f.w0 + 1 < geo.W;
                if (do_glob) {
                    u32x4 p00[NV], p01[NV], p10[NV], p11[NV];
                    far_corner_loads<NV>(vr, corner_offset(geo, t.n, f, es, chan_off), cs, rs, p00, p01, p10, p11);
                    // corners outside the image are zeros (zero-extended image)
                    const float t00 = (f.r0 && f.c0) ? corner_dot<T>(gov, p00) : 0.0f;
                    const float t01 = (f.r0 && f.c1) ? corner_dot<T>(gov, p01) : 0.0f;
                    const float t10 = (f.r1 && f.c0) ? corner_dot<T>(gov, p10) : 0.0f;
                    const float t11 = (f.r1 && f.c1) ? corner_dot<T>(gov, p11) : 0.0f;
                    float gm, gw, gh;
                    sample_grads(f.lh, f.lw, t00, t01, t10, t11, gm, gw, gh);
                    gm = pixel_sum(gm, lanes);
                    gw = pixel_sum(gw, lanes);
                    gh = pixel_sum(gh, lanes);
                    if (chunk == 0) {
                        const float sm = geo.scale * m;
                        grow[2 * k] = sm * gw;
                        grow[2 * k + 1] = sm * gh;
                        grow[2 * a.K + k] = gm;
                    }
                }
                if (do_atom) {
                    masked_weights(f, m, w00, w01, w10, w11);
                    // negative rows or columns wrap; only corners inside the
                    // image, which have non-zero weights, are written
                    cbase = gv_base + (unsigned)f.h0 * grs + (unsigned)f.w0 * gcs;
                }
            }
            // the prepared samples, one per pixel and group (its first lane)
            unsigned long long pend = __ballot(do_atom && chunk == 0);
            while (pend) {
                const int src = (int)__builtin_ctzll(pend);
                pend &= pend - 1;
                const float s00 = __builtin_bit_cast(float, __builtin_amdgcn_readlane(__builtin_bit_cast(int, w00), src));
                const float s01 = __builtin_bit_cast(float, __builtin_amdgcn_readlane(__builtin_bit_cast(int, w01), src));
                const float s10 = __builtin_bit_cast(float, __builtin_amdgcn_readlane(__builtin_bit_cast(int, w10), src));
                const float s11 = __builtin_bit_cast(float, __builtin_amdgcn_readlane(__builtin_bit_cast(int, w11), src));
                const unsigned sb = (unsigned)__builtin_amdgcn_readlane((int)cbase, src);
                // grad_output channel my_c of the sample's pixel and group
                unsigned gbits = 0u;
                for (int j = 0; j < lanes; ++j) {
#pragma unroll
                    for (int d = 0; d < 4 * NV; ++d) {
                        const unsigned x = gov[d >> 2][d & 3];
                        const unsigned y = (unsigned)__builtin_amdgcn_readlane((int)x, src + j);
                        gbits = (j == my_lane && d == my_dw) ? y : gbits;
                    }
                }
                float gval;
                if constexpr (es == 4)
                    gval = __builtin_bit_cast(float, gbits);
                else
                    gval = Store<T>::from_bits((my_c & 1) ? gbits >> 16 : gbits);
                const unsigned my_off = sb + 4u * (unsigned)my_c;
                for (int c0 = 0; c0 < 4; c0 += per_instr) {
                    const int corner = corner0 + c0;
                    if (corner < 4) {
                        const float w = corner == 0 ? s00 : corner == 1 ? s01 : corner == 2 ? s10 : s11;
                        if (w != 0.0f)
                            dcnv4_buffer_atomic_fadd(
                                w * gval, gr, (int)(my_off + (unsigned)(corner >> 1) * grs + (unsigned)(corner & 1) * gcs),
                                0, 0);
                    }
                }
            }
        }
    }
    if (SM && writer) {
        // gradients with respect to the logits: p_k * (g_k - sum_j p_j g_j),
        // with g_k = dL/dp_k
        float sdot = 0.0f;
#pragma unroll
        for (int k = 0; k < KMAX; ++k)
            sdot = k < a.K ? __builtin_fmaf(msk[k], grow[2 * a.K + k], sdot) : sdot;
#pragma unroll
        for (int k = 0; k < KMAX; ++k)
            if (k < a.K)
                grow[2 * a.K + k] = msk[k] * (grow[2 * a.K + k] - sdot);
    }
    __syncthreads();

    // write-back: pixel (ry, rx) of the tile holds the run of gb * 3K
    // entries from element t.g * 3K of its offset_mask row; consecutive
    // threads take consecutive dwords of a run.  The block of group 0 also
    // zeroes the padding entries.
    {
        const __amdgpu_buffer_rsrc_t r = rsrc(a.gom, a.om_bytes);
        const int rows = min(a.th, geo.Ho - t.oy0), cols = min(a.tw, geo.Wo - t.ox0);
        const int run = a.gb * 3 * a.K;
        const unsigned pbytes = (unsigned)(a.P * es);
        const unsigned run0 = (unsigned)(t.g * 3 * a.K * es);
        const unsigned tile0 = (unsigned)((t.n * geo.Ho + t.oy0) * geo.Wo + t.ox0);
        const float *src = reinterpret_cast<const float *>(lds);
        auto pixel_off = [&](int pq) -> int {   // -1 for a tile column outside the image
            const int ry = (int)divm((unsigned)pq, a.tw_magic), rx = pq - ry * a.tw;
            return rx < cols ? (int)((tile0 + (unsigned)(ry * geo.Wo + rx)) * pbytes) : -1;
        };
        // one entry per dword (fp32), two 16-bit entries per dword where the
        // runs start on even elements, else one 16-bit store per entry
        const bool pairs = es == 2 && run % 2 == 0 && (t.g * 3 * a.K) % 2 == 0;
        if (!pairs) {
            const int total = rows * a.tw * run;
            for (int j = threadIdx.x; j < total; j += blockDim.x) {
                const int pq = (int)divm((unsigned)j, a.run_magic);
                const int i = j - pq * run;
                const int po = pixel_off(pq);
                if (po < 0)
                    continue;
                const unsigned off = (unsigned)po + run0 + (unsigned)(i * es);
                if constexpr (es == 4)
                    __builtin_amdgcn_raw_buffer_store_b32(__builtin_bit_cast(unsigned, src[j]), r, off, 0, 0);
                else
                    __builtin_amdgcn_raw_buffer_store_b16(__builtin_bit_cast(unsigned short, Store<T>::make(src[j])),
                                                          r, off, 0, 0);
            }
        } else if constexpr (es == 2) {
            const int half = run >> 1;
            const int total = rows * a.tw * half;
            for (int j = threadIdx.x; j < total; j += blockDim.x) {
                const int pq = (int)divm((unsigned)j, a.half_magic);
                const int i = j - pq * half;
                const int po = pixel_off(pq);
                if (po < 0)
                    continue;
                const float lo = src[pq * run + 2 * i], hi = src[pq * run + 2 * i + 1];
                const unsigned w = (unsigned)__builtin_bit_cast(unsigned short, Store<T>::make(lo)) |
                                   ((unsigned)__builtin_bit_cast(unsigned short, Store<T>::make(hi)) << 16);
                __builtin_amdgcn_raw_buffer_store_b32(w, r, (unsigned)po + run0 + 4u * (unsigned)i, 0, 0);
            }
        }
        const int npad = a.P - a.G * 3 * a.K;
        if (t.g == 0 && npad > 0) {
            const unsigned pad0 = (unsigned)(a.G * 3 * a.K * es);
            const int total = rows * a.tw * npad;
            for (int j = threadIdx.x; j < total; j += blockDim.x) {
                const int pq = (int)divm((unsigned)j, a.npad_magic);
                const int i = j - pq * npad;
                const int po = pixel_off(pq);
                if (po < 0)
                    continue;
                const unsigned off = (unsigned)po + pad0 + (unsigned)(i * es);
                if constexpr (es == 4)
                    __builtin_amdgcn_raw_buffer_store_b32(0u, r, off, 0, 0);
                else
                    __builtin_amdgcn_raw_buffer_store_b16((unsigned short)0, r, off, 0, 0);
            }
        }
    }
}

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
        return dp == 16 ? offsets_for<_Float16, 16>(small_k, sm) : dp == 8 ? offsets_for<_Float16, 8>(small_k, sm)
                                                                            : nullptr;
    case DCNV4_BF16:
        return dp == 16 ? offsets_for<bf16_t, 16>(small_k, sm) : dp == 8 ? offsets_for<bf16_t, 8>(small_k, sm)
                                                                          : nullptr;
    default:
        return nullptr;
    }
}

}  // namespace tiled
}  // namespace dcnv4
