// Internal interface between the flash deformable attention C-ABI layer
// (fdattn_api.cpp) and its HIP kernels (fdattn_kernels.hip).  Not part of
// the ABI.
#pragma once

#include <hip/hip_runtime.h>

#include "flash_deform_attn.h"

#include <cstdint>

namespace fdattn {

constexpr int kMaxLevels = 16;
constexpr int kMaxPoints = 128;   // L*K
constexpr int kThreads = 256;     // threads per block, both kernels

// A validated call for the images [0, N) of one launch.  Every byte offset
// inside one launch's value and grad_value buffers fits in 31 bits.
struct Problem {
    int N, S, Q, M, D, K, L, P;
    int dtype, elem;
    int lvl_h[kMaxLevels], lvl_w[kMaxLevels], lvl_start[kMaxLevels];
};

// Enqueue the forward / backward for images [0, p.N) (pointers already
// offset to the launch's first image).  The backward sorts the samples in
// `workspace` (workspace_bytes(p) bytes, 16-byte aligned) and gathers
// grad_value; with workspace == nullptr it zero-fills grad_value and adds to
// it with device atomics.  Return hipError_t.
size_t workspace_bytes(const Problem &p);

hipError_t launch_forward(const Problem &p, const void *value, const void *loc_attn, void *output,
                          hipStream_t stream);
hipError_t launch_backward(const Problem &p, const void *value, const void *loc_attn, const void *grad_output,
                           float *grad_value, void *grad_loc_attn, void *workspace, hipStream_t stream);

// flash_deform_attn_backward_noalloc: its workspace is a library-owned
// device array of this many bytes per device (fdattn_noalloc.hip).
constexpr size_t kNoAllocScratchBytes = FLASH_DEFORM_ATTN_NOALLOC_SCRATCH_BYTES;
// Device address of that array on the current device, looked up on the
// first call per device (hipGetSymbolAddress) and kept; no allocation.
hipError_t noalloc_scratch(void **ptr);

}  // namespace fdattn
