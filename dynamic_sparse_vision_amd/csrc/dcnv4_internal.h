// Internal interface between the C-ABI layer (dcnv4_api.cpp) and the HIP
// kernels (dcnv4_kernels.hip: general path; dcnv4_tiled_*.hip: LDS-tiled
// path).  Not installed; not part of the ABI.
#pragma once

#include <hip/hip_runtime.h>

#include <cstddef>
#include <cstdint>

namespace dcnv4 {

namespace dev {
struct Geom;
}

// A fully validated call.  All sizes are positive and every derived byte
// count of one image fits in 31 bits.
struct Problem {
    int N, H, W, Ho, Wo;
    int kh, kw, sh, sw, ph, pw, dh, dw;
    int G, Cg, C, K, P;
    int remove_center;
    int softmax;       // 1: masks are logits normalised over the K points
    int dtype;         // enum dcnv4_dtype
    int elem;          // bytes per element of the storage dtype
    float offset_scale;
};

// General path: a block covers `pix_per_block` consecutive output pixels
// (in (n, ho, wo) order) and all of their groups; each (pixel, group) is
// handled by `lanes` threads of `dp` channels each.
struct Plan {
    int dp;             // channels per thread
    int lanes;          // threads per (pixel, group) = Cg / dp
    int pix_per_block;
    int threads;        // pix_per_block * G * lanes
    int lds_bytes;
    int images_per_launch;
};

// Cell-tile blocks of the backward's grad_value kernel: threads (one per
// vertical pair of cells) and the bin counters of a tile ((ch + 1) * (cw + 1)
// < kCellBinSlots; the in-place scan takes four per thread).
#ifndef DCNV4_CELL_THREADS
#define DCNV4_CELL_THREADS 512
#endif
constexpr int kCellThreads = DCNV4_CELL_THREADS;
constexpr int kCellBinSlots = 2048;
static_assert(4 * kCellThreads >= kCellBinSlots, "scan covers the bins");

// Tiled path.  An output-tile block stages the value rows its samples can
// reach within a halo of R pixels of the tile's grid (an LDS region of at
// most rh x rw pixels); a sample whose footprint lies in the region reads
// its corners there.  The backward's grad_value cell tiles take the samples
// whose integer displacement floor(loc) - (integer grid position) is within
// Rc pixels on both axes; the grad_offset_mask kernel adds the others with
// device atomics.
struct TilePlan {
    // output tiles (forward, backward grad_offset_mask): th x tw pixels of
    // one image and gb groups; lanes threads of dp channels per pixel and group
    int dp, lanes, th, tw, threads;
    int gb;              // groups per block (their slices of a pixel are contiguous)
    int tiles_y, tiles_x;
    int R;               // halo of the LDS value region of an output tile
    int Rc;              // backward: near radius of the grad_value cell tiles
    int rh, rw;          // LDS value region, pixels (the largest of any block)
    int nvp;             // 16-byte vectors per region pixel (Cg * elem / 16)
    int ps;              // LDS pixel stride, 16-byte slots ((gb * nvp) rounded up to odd)
    int lds_bytes;       // total LDS of an output-tile block (value rows; the backward's
                         // gradient rows reuse it at the end)
    // cell tiles (backward grad_value): ch x cw input cells of one (image, group)
    int ch, cw;
    int ctiles_y, ctiles_x;
    int src_cap;         // source pixels per batch (whole source rows)
    int gps;             // LDS stride of a staged grad_output pixel, 16-byte slots
    int rec_offset;      // LDS byte offset of the sorted sample records
    int gs_offset;       // LDS byte offset of the staged grad_output rows
    int splat_lds_bytes; // total LDS of a cell-tile block
    int images_per_launch;
};

// Host-side planning (pure C++, no HIP calls).  Return a dcnv4_status.
int plan_forward(const Problem &p, Plan *plan);
int plan_backward(const Problem &p, Plan *plan);
// Return DCNV4_OK when the tiled path applies, DCNV4_ERR_UNSUPPORTED if not.
int plan_forward_tiled(const Problem &p, TilePlan *tp);
int plan_backward_tiled(const Problem &p, TilePlan *tp);

dev::Geom make_geom(const Problem &p);

// The per-thread last-HIP-error text behind dcnv4_last_hip_error(): cleared
// at the start of every entry point; hip_status() records a failure and
// returns DCNV4_ERR_HIP (DCNV4_OK for hipSuccess).
void clear_hip_error();
int hip_status(hipError_t e);

// Raise a kernel's dynamic LDS limit to `bytes` on the current device when
// above the default 64 KB (gfx950 has 160 KB per CU); done once per kernel
// and device.
hipError_t allow_dynamic_lds(const void *fn, size_t bytes);

// Enqueue kernels for images [0, p.N) of the given tensors (the caller has
// already offset the pointers).  Return hipError_t.
hipError_t launch_zero(void *p, size_t bytes, hipStream_t stream);
hipError_t launch_forward_general(const Problem &p, const Plan &plan, const void *value,
                                  const void *offset_mask, void *output, hipStream_t stream);
hipError_t launch_backward_general(const Problem &p, const Plan &plan, const void *value,
                                   const void *offset_mask, const void *grad_output, void *grad_value,
                                   void *grad_offset_mask, hipStream_t stream);
hipError_t launch_forward_tiled(const Problem &p, const TilePlan &tp, const void *value,
                                const void *offset_mask, void *output, hipStream_t stream);
hipError_t launch_backward_tiled(const Problem &p, const TilePlan &tp, const void *value,
                                 const void *offset_mask, const void *grad_output, void *grad_value,
                                 void *grad_offset_mask, hipStream_t stream);

}  // namespace dcnv4
