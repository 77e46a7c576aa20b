// Internal interface between the C-ABI layer (dcnv4_api.cpp) and the HIP
// kernels (dcnv4_kernels.hip).  Not installed; not part of the ABI.
#pragma once

#include <hip/hip_runtime.h>

#include <cstddef>
#include <cstdint>

namespace dcnv4 {

// A fully validated call.  All sizes are positive and every derived byte
// count of one image fits in 31 bits.
struct Problem {
    int N, H, W, Ho, Wo;
    int kh, kw, sh, sw, ph, pw, dh, dw;
    int G, Cg, C, K, P;
    int remove_center;
    int dtype;         // enum dcnv4_dtype
    int elem;          // bytes per element of the storage dtype
    float offset_scale;
};

// Launch plan shared by the forward and backward kernels: a block covers
// `pix_per_block` consecutive output pixels (in (n, ho, wo) order) and all
// of their groups; each (pixel, group) is handled by `lanes` threads of
// `dp` channels each.
struct Plan {
    int dp;             // channels per thread
    int lanes;          // threads per (pixel, group) = Cg / dp
    int pix_per_block;
    int threads;        // pix_per_block * G * lanes
    int lds_bytes;
    int images_per_launch;
};

// Host-side planning (pure C++, no HIP calls).  Returns a dcnv4_status.
int plan_forward(const Problem &p, Plan *plan);
int plan_backward(const Problem &p, Plan *plan);

// Enqueue the kernels for images [0, p.N) of the given tensors (the caller
// has already offset the pointers).  Return hipError_t.
hipError_t launch_forward(const Problem &p, const Plan &plan, const void *value,
                          const void *offset_mask, void *output, hipStream_t stream);
hipError_t launch_backward(const Problem &p, const Plan &plan, const void *value,
                           const void *offset_mask, const void *grad_output, void *grad_value,
                           void *grad_offset_mask, hipStream_t stream);

}  // namespace dcnv4
